// kda_api.hip — host side of libkda.so: argument validation, workspace
// sizing and kernel launches for the C ABI declared in include/kda.h.
// Nothing is enqueued before every check has passed.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Alignment each pointer needs for the loads and stores the kernels issue on
// it: q, k, v, per-key alpha and every state are moved in 16-byte vectors
// (fp32 q/k/v and states) or 8-byte vectors (bf16 q/k/v in the decode step);
// scalar alpha, beta and o are moved one fp32 at a time; cu_seqlens in int64.
struct PtrReq {
  const void* p;
  uintptr_t align;
  const char* name;
};
int check_align(const PtrReq* reqs, int n) {
  for (int i = 0; i < n; ++i)
    if (reqs[i].p && !aligned(reqs[i].p, reqs[i].align))
      return fail(KDA_ERR_ALIGN, "%s (%p) must be %u-byte aligned", reqs[i].name, reqs[i].p,
                  (unsigned)reqs[i].align);
  return KDA_OK;
}

constexpr int64_t kChunk = 64;
constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int check_shape(const kda_shape* s) {
  if (!s) return fail(KDA_ERR_ARG, "shape is NULL");
  if (s->num_heads <= 0) return fail(KDA_ERR_SHAPE, "num_heads must be positive (got %d)", s->num_heads);
  if (s->d_k != s->d_v || (s->d_k != 64 && s->d_k != 128))
    return fail(KDA_ERR_SHAPE, "d_k = d_v in {64, 128} required (got d_k=%d d_v=%d)", s->d_k, s->d_v);
  if (s->qkv_dtype != KDA_BF16 && s->qkv_dtype != KDA_F32)
    return fail(KDA_ERR_ARG, "qkv_dtype must be KDA_BF16 or KDA_F32 (got %d)", s->qkv_dtype);
  if (s->gate != KDA_GATE_SCALAR && s->gate != KDA_GATE_PER_KEY)
    return fail(KDA_ERR_ARG, "gate must be KDA_GATE_SCALAR or KDA_GATE_PER_KEY (got %d)", s->gate);
  return KDA_OK;
}

// cu_seqlens: cu[0] == 0, nondecreasing, every length fits int32.
int check_cu(int32_t num_seqs, const int64_t* cu) {
  if (num_seqs < 0) return fail(KDA_ERR_ARG, "num_seqs must be >= 0 (got %d)", num_seqs);
  if (!cu) return fail(KDA_ERR_ARG, "cu_seqlens_host is NULL");
  if (cu[0] != 0) return fail(KDA_ERR_SHAPE, "cu_seqlens[0] must be 0 (got %lld)", (long long)cu[0]);
  for (int32_t n = 0; n < num_seqs; ++n) {
    const int64_t len = cu[n + 1] - cu[n];
    if (len < 0) return fail(KDA_ERR_SHAPE, "cu_seqlens decreases at index %d", n + 1);
    if (len > INT32_MAX - kChunk) return fail(KDA_ERR_SHAPE, "sequence %d is too long", n);
  }
  return KDA_OK;
}

int64_t snapshot_slots(int32_t num_seqs, const int64_t* cu, int64_t interval) {
  if (interval <= 0) return 0;
  int64_t total = 0;
  for (int32_t n = 0; n < num_seqs; ++n) total += (cu[n + 1] - cu[n]) / interval;
  return total;
}

// The snapshots buffer may be device memory or pinned host memory (then the
// kernels write the states over the bus while the prefill runs). Resolves
// the address the kernels use; pageable host memory is rejected.
int resolve_snapshots(float* p, float** dev_p) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(KDA_ERR_ARG, "snapshots (%p) is neither device memory nor pinned host memory", (void*)p);
  }
  if (attr.type == hipMemoryTypeHost) {
    if (!attr.devicePointer)
      return fail(KDA_ERR_ARG, "snapshots (%p): pinned host memory not mapped for the device", (void*)p);
    *dev_p = static_cast<float*>(attr.devicePointer);
    return KDA_OK;
  }
  if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) {
    *dev_p = p;
    return KDA_OK;
  }
  return fail(KDA_ERR_ARG, "snapshots (%p) is neither device memory nor pinned host memory", (void*)p);
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

// Work plan of one prefill call. Sequences longer than seg_chunks chunks are cut
// into segments (affine-map scan); seg_chunks == 0 runs every (sequence, head)
// chain in one workgroup.
struct PrefillPlan {
  int32_t seg_chunks, n_items;
  int32_t any_whole;   // segmented: some sequence is short enough to stay whole
  size_t items_off, first_off, maps_off, states_off, wu_off, bytes;
};

PrefillPlan plan_prefill(const kda_shape* s, int32_t num_seqs, const int64_t* cu,
                         int64_t segment_tokens, int cus) {
  PrefillPlan p{};
  int64_t total_chunks = 0, max_chunks = 0;
  for (int32_t n = 0; n < num_seqs; ++n) {
    const int64_t ch = (cu[n + 1] - cu[n] + kChunk - 1) / kChunk;
    total_chunks += ch;
    if (ch > max_chunks) max_chunks = ch;
  }
  int64_t seg = 0;
  if (segment_tokens > 0) {
    seg = segment_tokens / kChunk;
  } else if (segment_tokens < 0) {
    // automatic: split only when the (sequence, head) chains cannot fill the
    // device; aim at one workgroup per compute unit and at least 8 chunks per
    // segment.
    const int64_t units = (int64_t)num_seqs * s->num_heads;
    if (units < cus) {
      seg = (total_chunks * s->num_heads + cus - 1) / cus;
      if (seg < 8) seg = 8;
    }
  }
  if (seg >= max_chunks) seg = 0;   // no sequence would be split
  p.seg_chunks = (int32_t)seg;
  int64_t items = 0;
  for (int32_t n = 0; n < num_seqs; ++n) {
    const int64_t len = cu[n + 1] - cu[n];
    const int64_t st = seg * kChunk;
    const bool split = st > 0 && len > st;
    items += split ? (len + st - 1) / st : 1;
    if (!split) p.any_whole = 1;
  }
  p.n_items = (int32_t)items;
  const size_t H = (size_t)s->num_heads, DD = (size_t)s->d_k * s->d_v;
  size_t off = 0;
  p.items_off = off;
  off += round_up(sizeof(kda::PrefillItem) * (size_t)(items > 0 ? items : 1));
  p.first_off = off;
  off += round_up(sizeof(int32_t) * (size_t)(num_seqs > 0 ? num_seqs : 1));
  p.maps_off = off;
  if (seg > 0) off += round_up((size_t)items * H * 2 * DD * sizeof(float));
  p.states_off = off;
  if (seg > 0) off += round_up((size_t)items * H * DD * sizeof(float));
  p.wu_off = off;
  if (seg > 0) off += round_up((size_t)items * H * (size_t)seg * kda::wu_chunk_bytes(s->d_k));
  p.bytes = off;
  return p;
}

int check_prefill_args(const kda_shape* shape, int32_t num_seqs, const int64_t* cu,
                       int32_t chunk, int64_t interval, int64_t segment_tokens) {
  int rc = check_shape(shape);
  if (rc != KDA_OK) return rc;
  rc = check_cu(num_seqs, cu);
  if (rc != KDA_OK) return rc;
  if (chunk != kChunk) return fail(KDA_ERR_SHAPE, "chunk must be 64 (got %d)", chunk);
  if (interval < 0 || interval % kChunk != 0)
    return fail(KDA_ERR_SHAPE, "snapshot_interval must be 0 or a positive multiple of 64 (got %lld)",
                (long long)interval);
  if (segment_tokens < -1 || (segment_tokens > 0 && segment_tokens % kChunk != 0))
    return fail(KDA_ERR_SHAPE, "segment_tokens must be -1, 0 or a positive multiple of 64 (got %lld)",
                (long long)segment_tokens);
  return KDA_OK;
}

// Workspace of one backward call: the forward's own plan, its o / final
// scratch and the states after every 64 tokens, the chunk tables, then the
// per-(chunk, head) fp32 arrays of the backward kernels.
struct BackwardPlan {
  PrefillPlan fwd;
  int64_t n_chunks, n_snap, n_items;
  int32_t seg_chunks;
  size_t o_off, fin_off, snap_off, cb_off, sb_off, ib_off, maps_off, ends_off, ws_off, bytes;
};

BackwardPlan plan_backward(const kda_shape* s, int32_t num_seqs, const int64_t* cu, int cus) {
  BackwardPlan p{};
  p.fwd = plan_prefill(s, num_seqs, cu, -1, cus);
  int64_t max_chunks = 0;
  for (int32_t n = 0; n < num_seqs; ++n) {
    const int64_t ch = (cu[n + 1] - cu[n] + kChunk - 1) / kChunk;
    p.n_chunks += ch;
    if (ch > max_chunks) max_chunks = ch;
  }
  p.n_snap = snapshot_slots(num_seqs, cu, kChunk);
  // The reverse scan of the state gradient is sequential over the chunks of a
  // (sequence, head). When those chains cannot fill the device, sequences are
  // cut into segments (about two workgroups per compute unit, at least 8
  // chunks each) that are mapped in parallel, joined by a short scan over
  // segments, then run again from their true end gradients.
  int64_t seg = 0;
  if ((int64_t)num_seqs * s->num_heads < 2 * (int64_t)cus) {
    seg = (p.n_chunks * s->num_heads + 2 * (int64_t)cus - 1) / (2 * (int64_t)cus);
    if (seg < 8) seg = 8;
    if (seg >= max_chunks) seg = 0;
  }
  p.seg_chunks = (int32_t)seg;
  for (int32_t n = 0; n < num_seqs; ++n) {
    const int64_t ch = (cu[n + 1] - cu[n] + kChunk - 1) / kChunk;
    const int64_t it = seg > 0 ? (ch + seg - 1) / seg : 1;
    p.n_items += it > 0 ? it : 1;
  }
  const size_t H = (size_t)s->num_heads, D = (size_t)s->d_k, T = (size_t)cu[num_seqs];
  size_t off = round_up(p.fwd.bytes);
  p.o_off = off;
  off += round_up(T * H * D * sizeof(float));
  p.fin_off = off;
  off += round_up((size_t)num_seqs * H * D * D * sizeof(float));
  p.snap_off = off;
  off += round_up((size_t)p.n_snap * H * D * D * sizeof(float));
  p.cb_off = off;
  off += round_up(((size_t)num_seqs + 1) * sizeof(int64_t));
  p.sb_off = off;
  off += round_up(((size_t)num_seqs + 1) * sizeof(int64_t));
  p.ib_off = off;
  off += round_up(((size_t)num_seqs + 1) * sizeof(int64_t));
  p.maps_off = off;
  if (seg > 0) off += round_up((size_t)p.n_items * H * 2 * D * D * sizeof(float));
  p.ends_off = off;
  if (seg > 0) off += round_up((size_t)p.n_items * H * D * D * sizeof(float));
  p.ws_off = off;
  off += round_up((size_t)kda::bwd::floats(p.n_chunks * s->num_heads, s->d_k) * sizeof(float));
  p.bytes = off;
  return p;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_last_error(void) { return g_err; }

int kda_snapshot_count(int32_t num_seqs, const int64_t* cu_seqlens_host, int64_t interval,
                       int64_t* n_snap) {
  if (!n_snap) return fail(KDA_ERR_ARG, "n_snap is NULL");
  int rc = check_cu(num_seqs, cu_seqlens_host);
  if (rc != KDA_OK) return rc;
  if (interval < 0) return fail(KDA_ERR_SHAPE, "interval must be >= 0");
  *n_snap = snapshot_slots(num_seqs, cu_seqlens_host, interval);
  g_err[0] = '\0';
  return KDA_OK;
}

int kda_prefill_workspace_size(const kda_shape* shape, int32_t num_seqs,
                               const int64_t* cu_seqlens_host, int32_t chunk,
                               int64_t snapshot_interval, int64_t segment_tokens, size_t* bytes) {
  if (!bytes) return fail(KDA_ERR_ARG, "bytes is NULL");
  int rc = check_prefill_args(shape, num_seqs, cu_seqlens_host, chunk, snapshot_interval, segment_tokens);
  if (rc != KDA_OK) return rc;
  *bytes = plan_prefill(shape, num_seqs, cu_seqlens_host, segment_tokens,
                        segment_tokens < 0 ? device_cu_count() : 0).bytes;
  g_err[0] = '\0';
  return KDA_OK;
}

int kda_prefill_chunked(const kda_shape* shape, int32_t num_seqs,
                        const int64_t* cu_seqlens_host, const int64_t* cu_seqlens_dev,
                        int32_t chunk, int64_t snapshot_interval, int64_t segment_tokens,
                        const void* q, const void* k, const void* v,
                        const float* alpha, const float* beta,
                        const float* initial_state,
                        float* o, float* final_state, float* snapshots,
                        void* workspace, size_t workspace_bytes, void* hip_stream) {
  int rc = check_prefill_args(shape, num_seqs, cu_seqlens_host, chunk, snapshot_interval, segment_tokens);
  if (rc != KDA_OK) return rc;
  const int64_t T = cu_seqlens_host[num_seqs];
  const int64_t n_snap = snapshot_slots(num_seqs, cu_seqlens_host, snapshot_interval);
  if (num_seqs > 0 && !cu_seqlens_dev) return fail(KDA_ERR_ARG, "cu_seqlens_dev is NULL");
  if (T > 0 && (!q || !k || !v || !alpha || !beta || !o))
    return fail(KDA_ERR_ARG, "q, k, v, alpha, beta and o must be non-NULL when T > 0");
  if (num_seqs > 0 && !final_state) return fail(KDA_ERR_ARG, "final_state is NULL");
  if (n_snap > 0 && !snapshots)
    return fail(KDA_ERR_ARG, "snapshots is NULL but %lld snapshot slots are due", (long long)n_snap);
  const uintptr_t a_alpha = shape->gate == KDA_GATE_PER_KEY ? 16 : 4;
  const PtrReq reqs[] = {{q, 16, "q"}, {k, 16, "k"}, {v, 16, "v"}, {alpha, a_alpha, "alpha"},
                         {beta, 4, "beta"}, {initial_state, 16, "initial_state"}, {o, 16, "o"},
                         {final_state, 16, "final_state"},
                         {n_snap > 0 ? snapshots : nullptr, 16, "snapshots"},
                         {cu_seqlens_dev, 8, "cu_seqlens_dev"}, {workspace, 16, "workspace"}};
  rc = check_align(reqs, (int)(sizeof reqs / sizeof reqs[0]));
  if (rc != KDA_OK) return rc;
  const PrefillPlan plan = plan_prefill(shape, num_seqs, cu_seqlens_host, segment_tokens,
                                        segment_tokens < 0 ? device_cu_count() : 0);
  if (num_seqs > 0 && (!workspace || workspace_bytes < plan.bytes))
    return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", plan.bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (num_seqs == 0) {
    g_err[0] = '\0';
    return KDA_OK;
  }
  float* snaps_dev = nullptr;
  if (n_snap > 0) {
    rc = resolve_snapshots(snapshots, &snaps_dev);
    if (rc != KDA_OK) return rc;
  }

  kda::PrefillArgs a{};
  a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.init = initial_state;
  a.o = o; a.final_state = final_state; a.snapshots = snaps_dev;
  a.cu_dev = cu_seqlens_dev;
  a.num_seqs = num_seqs;
  a.H = shape->num_heads;
  a.interval = snapshot_interval;
  a.seg_chunks = plan.seg_chunks;
  a.n_items = plan.n_items;
  char* ws = static_cast<char*>(workspace);
  a.items = reinterpret_cast<kda::PrefillItem*>(ws + plan.items_off);
  a.seq_first_item = reinterpret_cast<int32_t*>(ws + plan.first_off);
  a.seg_maps = plan.seg_chunks > 0 ? reinterpret_cast<float*>(ws + plan.maps_off) : nullptr;
  a.seg_states = plan.seg_chunks > 0 ? reinterpret_cast<float*>(ws + plan.states_off) : nullptr;
  a.seg_wu = plan.seg_chunks > 0 ? static_cast<void*>(ws + plan.wu_off) : nullptr;
  a.any_whole = plan.any_whole;
  hipError_t e = kda::launch_prefill(a, shape->d_k, shape->qkv_dtype == KDA_BF16,
                                     shape->gate == KDA_GATE_PER_KEY,
                                     static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "prefill launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return KDA_OK;
}

int kda_decode_step(const kda_shape* shape, int32_t batch, const void* q, const void* k,
                    const void* v, const float* alpha, const float* beta, float* state,
                    float* o, void* hip_stream) {
  int rc = check_shape(shape);
  if (rc != KDA_OK) return rc;
  if (batch < 0) return fail(KDA_ERR_ARG, "batch must be >= 0 (got %d)", batch);
  if (batch == 0) {
    g_err[0] = '\0';
    return KDA_OK;
  }
  if ((int64_t)batch * shape->num_heads > INT32_MAX / 2)
    return fail(KDA_ERR_SHAPE, "batch * num_heads too large");
  if (!q || !k || !v || !alpha || !beta || !state || !o)
    return fail(KDA_ERR_ARG, "q, k, v, alpha, beta, state and o must be non-NULL");
  const uintptr_t a_qkv = shape->qkv_dtype == KDA_BF16 ? 8 : 16;
  const uintptr_t a_alpha = shape->gate == KDA_GATE_PER_KEY ? 16 : 4;
  const PtrReq reqs[] = {{q, a_qkv, "q"}, {k, a_qkv, "k"}, {v, 4, "v"}, {alpha, a_alpha, "alpha"},
                         {beta, 4, "beta"}, {state, 16, "state"}, {o, 4, "o"}};
  rc = check_align(reqs, (int)(sizeof reqs / sizeof reqs[0]));
  if (rc != KDA_OK) return rc;
  kda::DecodeArgs a{q, k, v, alpha, beta, state, o, batch, shape->num_heads};
  hipError_t e = kda::launch_decode(a, shape->d_k, shape->qkv_dtype == KDA_BF16,
                                    shape->gate == KDA_GATE_PER_KEY,
                                    static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "decode launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return KDA_OK;
}

int kda_decode_tokens(const kda_shape* shape, int32_t batch, int32_t n_tok, const void* q,
                      const void* k, const void* v, const float* alpha, const float* beta,
                      float* state, float* o, float* token_states, const int32_t* commit,
                      void* hip_stream) {
  int rc = check_shape(shape);
  if (rc != KDA_OK) return rc;
  if (batch < 0) return fail(KDA_ERR_ARG, "batch must be >= 0 (got %d)", batch);
  if (n_tok < 0) return fail(KDA_ERR_ARG, "n_tok must be >= 0 (got %d)", n_tok);
  if (batch == 0 || n_tok == 0) {
    g_err[0] = '\0';
    return KDA_OK;
  }
  if ((int64_t)batch * shape->num_heads > INT32_MAX / 2 ||
      (int64_t)batch * n_tok * shape->num_heads > INT32_MAX / 2)
    return fail(KDA_ERR_SHAPE, "batch * n_tok * num_heads too large");
  if (!q || !k || !v || !alpha || !beta || !state || !o)
    return fail(KDA_ERR_ARG, "q, k, v, alpha, beta, state and o must be non-NULL");
  const uintptr_t a_qkv = shape->qkv_dtype == KDA_BF16 ? 8 : 16;
  const uintptr_t a_alpha = shape->gate == KDA_GATE_PER_KEY ? 16 : 4;
  const PtrReq reqs[] = {{q, a_qkv, "q"}, {k, a_qkv, "k"}, {v, 4, "v"}, {alpha, a_alpha, "alpha"},
                         {beta, 4, "beta"}, {state, 16, "state"}, {o, 4, "o"},
                         {token_states, 16, "token_states"}, {commit, 4, "commit"}};
  rc = check_align(reqs, (int)(sizeof reqs / sizeof reqs[0]));
  if (rc != KDA_OK) return rc;
  kda::DecodeArgs a{q, k, v, alpha, beta, state, o, batch, shape->num_heads, n_tok, token_states, commit};
  hipError_t e = kda::launch_decode_tokens(a, shape->d_k, shape->qkv_dtype == KDA_BF16,
                                           shape->gate == KDA_GATE_PER_KEY,
                                           static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "decode launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return KDA_OK;
}

int kda_layer_front(const kda_shape* shape, int32_t num_seqs, const int64_t* cu_seqlens_host,
                    const int64_t* cu_seqlens_dev, const void* xq, const void* xk, const void* xv,
                    const float* conv_w, const void* conv_state_in, const float* alpha_logit,
                    float alpha_bias, const float* beta_logit, void* q, void* k, void* v, float* alpha,
                    float* beta, void* conv_state_out, void* hip_stream) {
  int rc = check_shape(shape);
  if (rc != KDA_OK) return rc;
  rc = check_cu(num_seqs, cu_seqlens_host);
  if (rc != KDA_OK) return rc;
  const int64_t T = cu_seqlens_host[num_seqs];
  if (num_seqs > 0 && !cu_seqlens_dev) return fail(KDA_ERR_ARG, "cu_seqlens_dev is NULL");
  if (T > 0 && (!xq || !xk || !xv || !conv_w || !alpha_logit || !beta_logit || !q || !k || !v || !alpha || !beta))
    return fail(KDA_ERR_ARG, "inputs, conv_w, gate logits and outputs must be non-NULL when T > 0");
  if (num_seqs > 0 && !conv_w) return fail(KDA_ERR_ARG, "conv_w is NULL");
  const uintptr_t a_alpha = shape->gate == KDA_GATE_PER_KEY ? 16 : 4;
  const PtrReq reqs[] = {{xq, 16, "xq"}, {xk, 16, "xk"}, {xv, 16, "xv"}, {conv_w, 16, "conv_w"},
                         {conv_state_in, 16, "conv_state_in"}, {alpha_logit, a_alpha, "alpha_logit"},
                         {beta_logit, 4, "beta_logit"}, {q, 16, "q"}, {k, 16, "k"}, {v, 16, "v"},
                         {alpha, a_alpha, "alpha"}, {beta, 4, "beta"}, {conv_state_out, 16, "conv_state_out"},
                         {cu_seqlens_dev, 8, "cu_seqlens_dev"}};
  rc = check_align(reqs, (int)(sizeof reqs / sizeof reqs[0]));
  if (rc != KDA_OK) return rc;
  // neighbouring workgroups read the 3 rows before their first token, and the
  // carried-state pass shifts within a sequence's slots: no output may be an input
  if ((q && (q == xq || q == xk || q == xv)) || (k && (k == xq || k == xk || k == xv)) ||
      (v && (v == xq || v == xk || v == xv)))
    return fail(KDA_ERR_ARG, "q, k, v must not alias xq, xk, xv");
  if (conv_state_out && conv_state_out == conv_state_in)
    return fail(KDA_ERR_ARG, "conv_state_out must not alias conv_state_in");
  kda::LayerFrontArgs a{};
  a.xq = xq; a.xk = xk; a.xv = xv; a.conv_w = conv_w; a.conv_state_in = conv_state_in;
  a.alpha_logit = alpha_logit; a.beta_logit = beta_logit; a.alpha_bias = alpha_bias;
  a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.conv_state_out = conv_state_out;
  a.cu = cu_seqlens_dev; a.num_seqs = num_seqs; a.H = shape->num_heads; a.T = T;
  if (num_seqs == 0) {
    g_err[0] = '\0';
    return KDA_OK;
  }
  hipError_t e = kda::launch_layer_front(a, shape->d_k, shape->qkv_dtype == KDA_BF16,
                                         shape->gate == KDA_GATE_PER_KEY, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "layer front launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return KDA_OK;
}

int kda_layer_back(const kda_shape* shape, int64_t num_tokens, const float* o, const float* g_logit,
                   const float* norm_w, float eps, int32_t out_dtype, void* out, void* hip_stream) {
  int rc = check_shape(shape);
  if (rc != KDA_OK) return rc;
  if (num_tokens < 0) return fail(KDA_ERR_ARG, "num_tokens must be >= 0");
  if (out_dtype != KDA_BF16 && out_dtype != KDA_F32)
    return fail(KDA_ERR_ARG, "out_dtype must be KDA_BF16 or KDA_F32 (got %d)", out_dtype);
  if (!(eps >= 0.f)) return fail(KDA_ERR_ARG, "eps must be >= 0");
  if (num_tokens == 0) {
    g_err[0] = '\0';
    return KDA_OK;
  }
  if (!o || !g_logit || !norm_w || !out) return fail(KDA_ERR_ARG, "o, g_logit, norm_w and out must be non-NULL");
  const PtrReq reqs[] = {{o, 16, "o"}, {g_logit, 16, "g_logit"}, {norm_w, 16, "norm_w"}, {out, 16, "out"}};
  rc = check_align(reqs, (int)(sizeof reqs / sizeof reqs[0]));
  if (rc != KDA_OK) return rc;
  kda::LayerBackArgs a{o, g_logit, norm_w, out, eps, num_tokens * shape->num_heads};
  hipError_t e = kda::launch_layer_back(a, shape->d_v, out_dtype == KDA_BF16, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "layer back launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return KDA_OK;
}

int kda_prefill_backward_workspace_size(const kda_shape* shape, int32_t num_seqs,
                                        const int64_t* cu_seqlens_host, size_t* bytes) {
  if (!bytes) return fail(KDA_ERR_ARG, "bytes is NULL");
  int rc = check_shape(shape);
  if (rc != KDA_OK) return rc;
  rc = check_cu(num_seqs, cu_seqlens_host);
  if (rc != KDA_OK) return rc;
  *bytes = plan_backward(shape, num_seqs, cu_seqlens_host, device_cu_count()).bytes;
  g_err[0] = '\0';
  return KDA_OK;
}

int kda_prefill_backward(const kda_shape* shape, int32_t num_seqs, const int64_t* cu_seqlens_host,
                         const int64_t* cu_seqlens_dev, const void* q, const void* k, const void* v,
                         const float* alpha, const float* beta, const float* initial_state, const float* d_o,
                         const float* d_final_state, float* dq, float* dk, float* dv, float* dalpha,
                         float* dbeta, float* d_initial_state, void* workspace, size_t workspace_bytes,
                         void* hip_stream) {
  int rc = check_shape(shape);
  if (rc != KDA_OK) return rc;
  rc = check_cu(num_seqs, cu_seqlens_host);
  if (rc != KDA_OK) return rc;
  const int64_t T = cu_seqlens_host[num_seqs];
  if (num_seqs > 0 && !cu_seqlens_dev) return fail(KDA_ERR_ARG, "cu_seqlens_dev is NULL");
  if (T > 0 && (!q || !k || !v || !alpha || !beta || !d_o || !dq || !dk || !dv || !dalpha || !dbeta))
    return fail(KDA_ERR_ARG, "inputs, d_o and the gradient outputs must be non-NULL when T > 0");
  const uintptr_t a_alpha = shape->gate == KDA_GATE_PER_KEY ? 16 : 4;
  const PtrReq reqs[] = {{q, 16, "q"}, {k, 16, "k"}, {v, 16, "v"}, {alpha, a_alpha, "alpha"},
                         {beta, 4, "beta"}, {initial_state, 16, "initial_state"}, {d_o, 4, "d_o"},
                         {d_final_state, 16, "d_final_state"}, {dq, 16, "dq"}, {dk, 16, "dk"}, {dv, 16, "dv"},
                         {dalpha, a_alpha, "dalpha"}, {dbeta, 4, "dbeta"}, {d_initial_state, 16, "d_initial_state"},
                         {cu_seqlens_dev, 8, "cu_seqlens_dev"}, {workspace, 16, "workspace"}};
  rc = check_align(reqs, (int)(sizeof reqs / sizeof reqs[0]));
  if (rc != KDA_OK) return rc;
  if (num_seqs == 0) {
    g_err[0] = '\0';
    return KDA_OK;
  }
  const BackwardPlan plan = plan_backward(shape, num_seqs, cu_seqlens_host, device_cu_count());
  if (!workspace || workspace_bytes < plan.bytes)
    return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", plan.bytes,
                workspace ? workspace_bytes : (size_t)0);
  char* ws = static_cast<char*>(workspace);
  const hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const bool bf16 = shape->qkv_dtype == KDA_BF16, pk = shape->gate == KDA_GATE_PER_KEY;

  // 1. the forward again, keeping the state after every 64 tokens
  kda::PrefillArgs f{};
  f.q = q; f.k = k; f.v = v; f.alpha = alpha; f.beta = beta; f.init = initial_state;
  f.o = reinterpret_cast<float*>(ws + plan.o_off);
  f.final_state = reinterpret_cast<float*>(ws + plan.fin_off);
  f.snapshots = plan.n_snap > 0 ? reinterpret_cast<float*>(ws + plan.snap_off) : nullptr;
  f.cu_dev = cu_seqlens_dev;
  f.num_seqs = num_seqs;
  f.H = shape->num_heads;
  f.interval = kChunk;
  f.seg_chunks = plan.fwd.seg_chunks;
  f.n_items = plan.fwd.n_items;
  f.items = reinterpret_cast<kda::PrefillItem*>(ws + plan.fwd.items_off);
  f.seq_first_item = reinterpret_cast<int32_t*>(ws + plan.fwd.first_off);
  f.seg_maps = plan.fwd.seg_chunks > 0 ? reinterpret_cast<float*>(ws + plan.fwd.maps_off) : nullptr;
  f.seg_states = plan.fwd.seg_chunks > 0 ? reinterpret_cast<float*>(ws + plan.fwd.states_off) : nullptr;
  f.seg_wu = plan.fwd.seg_chunks > 0 ? static_cast<void*>(ws + plan.fwd.wu_off) : nullptr;
  f.any_whole = plan.fwd.any_whole;
  hipError_t e = kda::launch_prefill(f, shape->d_k, bf16, pk, st);
  if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "backward: forward launch failed: %s", hipGetErrorString(e));

  // 2. the backward kernels
  kda::BackwardArgs b{};
  b.q = q; b.k = k; b.v = v; b.alpha = alpha; b.beta = beta; b.init = initial_state;
  b.d_o = d_o; b.d_final = d_final_state;
  b.dq = dq; b.dk = dk; b.dv = dv; b.dalpha = dalpha; b.dbeta = dbeta; b.d_init = d_initial_state;
  b.cu_dev = cu_seqlens_dev;
  b.num_seqs = num_seqs;
  b.H = shape->num_heads;
  b.n_chunks = plan.n_chunks;
  b.states = reinterpret_cast<const float*>(ws + plan.snap_off);
  b.chunk_base = reinterpret_cast<int64_t*>(ws + plan.cb_off);
  b.snap_base = reinterpret_cast<int64_t*>(ws + plan.sb_off);
  b.item_base = reinterpret_cast<int64_t*>(ws + plan.ib_off);
  b.seg_chunks = plan.seg_chunks;
  b.n_items = plan.n_items;
  b.seg_maps = plan.seg_chunks > 0 ? reinterpret_cast<float*>(ws + plan.maps_off) : nullptr;
  b.seg_end = plan.seg_chunks > 0 ? reinterpret_cast<float*>(ws + plan.ends_off) : nullptr;
  b.ws = reinterpret_cast<float*>(ws + plan.ws_off);
  e = kda::launch_backward(b, shape->d_k, bf16, pk, st);
  if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "backward launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return KDA_OK;
}

}  // extern "C"
