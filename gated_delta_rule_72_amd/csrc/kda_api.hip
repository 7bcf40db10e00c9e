// kda_api.hip — host side of libkda.so: argument validation, workspace
// sizing and kernel launches for the C ABI declared in include/kda.h.
// Nothing is enqueued before every check has passed.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

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

// d_k and d_v each 64 or 128; `square` additionally requires d_k = d_v (the
// backward pass and the layer front end).
int check_shape(const kda_shape* s, bool square = false) {
  if (!s) return fail(KDA_ERR_ARG, "shape is NULL");
  if (s->num_heads <= 0) return fail(KDA_ERR_SHAPE, "num_heads must be positive (got %d)", s->num_heads);
  if ((s->d_k != 64 && s->d_k != 128) || (s->d_v != 64 && s->d_v != 128))
    return fail(KDA_ERR_SHAPE, "d_k and d_v must each be 64 or 128 (got d_k=%d d_v=%d)", s->d_k, s->d_v);
  if (square && s->d_k != s->d_v)
    return fail(KDA_ERR_SHAPE, "this entry point needs d_k = d_v (got d_k=%d d_v=%d)", s->d_k, s->d_v);
  if (s->qkv_dtype != KDA_BF16 && s->qkv_dtype != KDA_F32)
    return fail(KDA_ERR_ARG, "qkv_dtype must be KDA_BF16 or KDA_F32 (got %d)", s->qkv_dtype);
  if (s->gate != KDA_GATE_SCALAR && s->gate != KDA_GATE_PER_KEY)
    return fail(KDA_ERR_ARG, "gate must be KDA_GATE_SCALAR or KDA_GATE_PER_KEY (got %d)", s->gate);
  // the kernels form element and byte offsets within one 64-token chunk of a
  // [T][H][128] fp32 tensor in 32 bits
  if ((int64_t)s->num_heads * 128 * 64 * 4 > INT32_MAX)
    return fail(KDA_ERR_SHAPE, "num_heads must be at most 65535 (got %d)", s->num_heads);
  return KDA_OK;
}

// Byte ranges [p, p + n) that must not overlap (an output against the inputs).
struct Range {
  const void* p;
  size_t n;
  const char* name;
};
bool overlap(const Range& a, const Range& b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.n && b0 < a0 + a.n;
}
int check_disjoint(const Range& out, const Range* ins, int n_in) {
  for (int i = 0; i < n_in; ++i)
    if (overlap(out, ins[i]))
      return fail(KDA_ERR_ARG, "%s overlaps %s (outputs must not alias inputs)", out.name, ins[i].name);
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
  int32_t one_seq;     // one sequence: the kernels form the work items themselves
  int64_t one_tok0, one_len;
  int64_t whole_tokens;  // segmented: tokens of the sequences that stay whole
  size_t items_off, first_off, maps_off, states_off, wu_off, bytes;
};

// The kernels run square heads, d = d_k = d_v. Rows of the state evolve
// independently (each row sees only its own value channel), which gives the
// two rectangular shapes:
//   d_v = 2 d_k: every head's d_v rows split into two value heads of d_k rows
//     (H' = 2H, qk_shift = 1; v, o and the states are laid out alike);
//   d_k = 2 d_v: the values and states are padded with zero rows to d_k in
//     the workspace (zero rows stay zero), the outputs copied back.
struct Geometry {
  int d;          // kernel head size
  int H;          // kernel head count
  int qk_shift;
  bool pad;       // d_k = 2 d_v
};
Geometry geometry(const kda_shape* s) {
  if (s->d_v == 2 * s->d_k) return {s->d_k, 2 * s->num_heads, 1, false};
  return {s->d_k, s->num_heads, 0, s->d_k == 2 * s->d_v};
}

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
    if (!split) {
      p.any_whole = 1;
      p.whole_tokens += len;
    }
  }
  p.n_items = (int32_t)items;
  if (num_seqs == 1) {
    p.one_seq = 1;
    p.one_tok0 = cu[0];
    p.one_len = cu[1] - cu[0];
  }
  const size_t H = (size_t)s->num_heads, DD = (size_t)s->d_k * s->d_k;
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

// The kernels' plan (square heads of the geometry) followed, for padded heads,
// by the padded values, initial state, o, final state and snapshots.
struct FullPlan {
  Geometry geo;
  PrefillPlan kern;
  size_t v_off, init_off, o_off, fin_off, snap_off, bytes;
};
FullPlan plan_full(const kda_shape* s, int32_t num_seqs, const int64_t* cu, int64_t interval,
                   int64_t segment_tokens, int cus) {
  FullPlan f{};
  f.geo = geometry(s);
  kda_shape ks = *s;
  ks.num_heads = f.geo.H;
  ks.d_k = ks.d_v = f.geo.d;
  f.kern = plan_prefill(&ks, num_seqs, cu, segment_tokens, cus);
  size_t off = f.kern.bytes;
  if (f.geo.pad) {
    const size_t T = (size_t)cu[num_seqs], H = (size_t)s->num_heads, d = (size_t)f.geo.d;
    const size_t es = s->qkv_dtype == KDA_BF16 ? 2 : 4, DD = d * d * sizeof(float);
    f.v_off = off;
    off += round_up(T * H * d * es);
    f.init_off = off;
    off += round_up((size_t)num_seqs * H * DD);
    f.o_off = off;
    off += round_up(T * H * d * sizeof(float));
    f.fin_off = off;
    off += round_up((size_t)num_seqs * H * DD);
    f.snap_off = off;
    off += round_up((size_t)snapshot_slots(num_seqs, cu, interval) * H * DD);
  }
  f.bytes = off;
  return f;
}

// Workspace of kda_layer_prefill: the prefill's own plan, then the 16-byte sink
// of the back end fused into pass 3, or, where it does not apply, an fp32 o
// [T, H, d] that the separate back-end kernel reads.
struct LayerPlan {
  FullPlan pre;
  bool fused;
  size_t aux_off, bytes;
};
LayerPlan plan_layer(const kda_shape* s, int32_t num_seqs, const int64_t* cu, int64_t interval,
                     int64_t segment_tokens, int cus) {
  LayerPlan l{};
  l.pre = plan_full(s, num_seqs, cu, interval, segment_tokens, cus);
  // pass 3 carries the fused back end in two forms, the scalar gate at d = 128
  // and the per-key (KDA) gate at d = 64, both with bf16 inputs; it runs the
  // segments of split sequences, so every sequence with tokens must be split
  // (empty ones only take their final state from the other pass)
  const bool form = s->qkv_dtype == KDA_BF16 && ((s->d_k == 128 && s->gate == KDA_GATE_SCALAR) ||
                                                 (s->d_k == 64 && s->gate == KDA_GATE_PER_KEY));
  l.fused = form && l.pre.kern.seg_chunks > 0 && l.pre.kern.whole_tokens == 0;
  l.aux_off = round_up(l.pre.bytes);
  l.bytes = l.aux_off + (l.fused ? kAlign : round_up((size_t)cu[num_seqs] * s->num_heads * s->d_v * sizeof(float)));
  return l;
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
  bool s0_in_place;   // one sequence: the forward's 64-token states land in the chunk-start array
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
  // With one sequence, the state after 64 (j + 1) tokens is the start state
  // of chunk j + 1, unit (j + 1) H + h of the backward's chunk-start array:
  // the forward writes it there and needs no state slots of its own.
  p.s0_in_place = num_seqs == 1;
  p.snap_off = off;
  if (!p.s0_in_place) off += round_up((size_t)p.n_snap * H * D * D * sizeof(float));
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

// Every host check of a prefill call, before anything is planned or enqueued.
int validate_prefill(const kda_shape* shape, int32_t num_seqs, const int64_t* cu_seqlens_host,
                     const int64_t* cu_seqlens_dev, int32_t chunk, int64_t snapshot_interval,
                     int64_t segment_tokens, const void* q, const void* k, const void* v,
                     const float* alpha, const float* beta, const float* initial_state, const void* o,
                     const float* final_state, const float* snapshots, const void* workspace,
                     size_t workspace_bytes, size_t o_elem = 4, const char* o_name = "o") {
  int rc = check_prefill_args(shape, num_seqs, cu_seqlens_host, chunk, snapshot_interval, segment_tokens);
  if (rc != KDA_OK) return rc;
  const int64_t T = cu_seqlens_host[num_seqs];
  const int64_t n_snap = snapshot_slots(num_seqs, cu_seqlens_host, snapshot_interval);
  if (num_seqs > 0 && !cu_seqlens_dev) return fail(KDA_ERR_ARG, "cu_seqlens_dev is NULL");
  if (T > 0 && (!q || !k || !v || !alpha || !beta || !o))
    return fail(KDA_ERR_ARG, "q, k, v, alpha, beta and %s must be non-NULL when T > 0", o_name);
  if (num_seqs > 0 && !final_state) return fail(KDA_ERR_ARG, "final_state is NULL");
  if (n_snap > 0 && !snapshots)
    return fail(KDA_ERR_ARG, "snapshots is NULL but %lld snapshot slots are due", (long long)n_snap);
  const uintptr_t a_alpha = shape->gate == KDA_GATE_PER_KEY ? 16 : 4;
  const PtrReq reqs[] = {{q, 16, "q"}, {k, 16, "k"}, {v, 16, "v"}, {alpha, a_alpha, "alpha"},
                         {beta, 4, "beta"}, {initial_state, 16, "initial_state"}, {o, 16, o_name},
                         {final_state, 16, "final_state"},
                         {n_snap > 0 ? snapshots : nullptr, 16, "snapshots"},
                         {cu_seqlens_dev, 8, "cu_seqlens_dev"}, {workspace, 16, "workspace"}};
  rc = check_align(reqs, (int)(sizeof reqs / sizeof reqs[0]));
  if (rc != KDA_OK) return rc;
  {
    // o, the final states and the snapshots are written while the inputs are
    // still read: none may overlap an input (final_state may only be
    // initial_state itself) or another output
    const size_t H = (size_t)shape->num_heads, es = shape->qkv_dtype == KDA_BF16 ? 2 : 4;
    const size_t tokh = (size_t)T * H, st = (size_t)shape->d_k * shape->d_v * sizeof(float);
    const size_t a_n = tokh * (shape->gate == KDA_GATE_PER_KEY ? (size_t)shape->d_k : 1) * sizeof(float);
    const Range ins[] = {{q, tokh * shape->d_k * es, "q"}, {k, tokh * shape->d_k * es, "k"},
                         {v, tokh * shape->d_v * es, "v"}, {alpha, a_n, "alpha"},
                         {beta, tokh * sizeof(float), "beta"},
                         {initial_state, (size_t)num_seqs * H * st, "initial_state"},
                         {cu_seqlens_dev, ((size_t)num_seqs + 1) * sizeof(int64_t), "cu_seqlens_dev"},
                         {workspace, workspace_bytes, "workspace"}};
    const int n_in = (int)(sizeof ins / sizeof ins[0]);
    const Range ro{o, tokh * shape->d_v * o_elem, o_name};
    const Range rf{final_state, (size_t)num_seqs * H * st, "final_state"};
    const Range rs{n_snap > 0 ? snapshots : nullptr, (size_t)n_snap * H * st, "snapshots"};
    if ((rc = check_disjoint(ro, ins, n_in)) != KDA_OK) return rc;
    if (final_state != initial_state && (rc = check_disjoint(rf, ins, n_in)) != KDA_OK) return rc;
    if (final_state == initial_state && (rc = check_disjoint(rf, ins + 6, n_in - 6)) != KDA_OK) return rc;
    if ((rc = check_disjoint(rs, ins, n_in)) != KDA_OK) return rc;
    const Range outs[] = {ro, rf};
    if ((rc = check_disjoint(rs, outs, 2)) != KDA_OK) return rc;
    if ((rc = check_disjoint(ro, outs + 1, 1)) != KDA_OK) return rc;
  }
  return KDA_OK;
}

// ---- static scratch of the allocation-free prefill ------------------------------
// kda_prefill_chunked_noalloc takes its work table from this array instead of a
// caller's workspace. Each GPU holds its own copy for the life of the process;
// host code uses the device address that hipGetSymbolAddress returns for the
// current device, never the array's name (a host-side stand-in).
constexpr size_t kScratchBytes = 1u << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; NULL with the HIP error's text
// in g_err if the lookup fails.
void* scratch_address() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    fail(KDA_ERR_DEVICE, "no current HIP device (or device index above %d)", kMaxDevices - 1);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      fail(KDA_ERR_DEVICE, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
      return nullptr;
    }
    addr[dev] = p;
  }
  return addr[dev];
}

// Heads are independent in the backward. When the plan for all heads would
// need more than kBackwardBudget bytes of workspace, the heads run in groups
// of Hg: each group's inputs are gathered into contiguous [.., Hg, ..]
// slices of the workspace, the backward runs on them, and the gradients are
// scattered back. 96 GiB, a third of an MI355X's HBM, keeps the long-prefill
// shape (T = 262144, H = 16, d = 128: about 75 GB) in one group and leaves room
// for the caller's tensors beside the largest packs.
constexpr size_t kBackwardBudget = (size_t)96 << 30;
// KDA_BACKWARD_BUDGET_BYTES in the environment lowers (or raises) the budget,
// read at every call (tests force small groups with it).
size_t backward_budget() {
  const char* e = getenv("KDA_BACKWARD_BUDGET_BYTES");
  if (!e || !*e) return kBackwardBudget;
  const unsigned long long v = strtoull(e, nullptr, 10);
  return v > 0 ? (size_t)v : kBackwardBudget;
}
struct GroupedBackward {
  int Hg, groups;
  BackwardPlan plan;                       // of one group of Hg heads
  // gathered inputs and group outputs (offsets into the workspace)
  size_t q_off, k_off, v_off, a_off, b_off, init_off, do_off, df_off;
  size_t dq_off, dk_off, dv_off, da_off, db_off, di_off, bytes;
};
GroupedBackward plan_backward_grouped(const kda_shape* s, int32_t num_seqs, const int64_t* cu, int cus) {
  GroupedBackward g{};
  const int H = s->num_heads;
  const size_t budget = backward_budget();
  for (int groups = 1; groups <= H; ++groups) {
    const int Hg = (H + groups - 1) / groups;
    if (groups > 1 && (H + Hg - 1) / Hg != groups) continue;     // same Hg as fewer groups
    kda_shape gs = *s;
    gs.num_heads = Hg;
    g.Hg = Hg;
    g.groups = groups;
    g.plan = plan_backward(&gs, num_seqs, cu, cus);
    size_t plan_bytes = g.plan.bytes;
    if (H % Hg) {                          // the last, smaller group plans its own segments
      gs.num_heads = H % Hg;
      const size_t last = plan_backward(&gs, num_seqs, cu, cus).bytes;
      plan_bytes = last > plan_bytes ? last : plan_bytes;
    }
    size_t off = round_up(plan_bytes);
    if (groups > 1) {
      const size_t T = (size_t)cu[num_seqs], d = (size_t)s->d_k, N = (size_t)num_seqs;
      const size_t es = s->qkv_dtype == KDA_BF16 ? 2 : 4;
      const size_t a_el = s->gate == KDA_GATE_PER_KEY ? d : 1, st = N * Hg * d * d * 4;
      auto take = [&](size_t& o, size_t n) { o = off; off += round_up(n); };
      take(g.q_off, T * Hg * d * es); take(g.k_off, T * Hg * d * es); take(g.v_off, T * Hg * d * es);
      take(g.a_off, T * Hg * a_el * 4); take(g.b_off, T * Hg * 4); take(g.init_off, st);
      take(g.do_off, T * Hg * d * 4); take(g.df_off, st);
      take(g.dq_off, T * Hg * d * 4); take(g.dk_off, T * Hg * d * 4); take(g.dv_off, T * Hg * d * 4);
      take(g.da_off, T * Hg * a_el * 4); take(g.db_off, T * Hg * 4); take(g.di_off, st);
    }
    g.bytes = off;
    if (g.bytes <= budget || Hg == 1) break;
  }
  return g;
}

// One backward launch sequence (forward recompute, then the backward kernels)
// on H = shape->num_heads heads whose tensors start at the given pointers.
int run_backward(const kda_shape* shape, int32_t num_seqs, const int64_t* cu_seqlens_dev, const BackwardPlan& plan,
                 const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                 const float* initial_state, const float* d_o, const float* d_final_state, float* dq, float* dk,
                 float* dv, float* dalpha, float* dbeta, float* d_initial_state, char* ws, hipStream_t st) {
  const bool bf16 = shape->qkv_dtype == KDA_BF16, pk = shape->gate == KDA_GATE_PER_KEY;
  // 1. the forward again, keeping the state after every 64 tokens
  kda::PrefillArgs f{};
  f.q = q; f.k = k; f.v = v; f.alpha = alpha; f.beta = beta; f.init = initial_state;
  f.o = reinterpret_cast<float*>(ws + plan.o_off);
  f.final_state = reinterpret_cast<float*>(ws + plan.fin_off);
  // (one sequence: straight into the chunk-start array from its unit H on; a
  // state after the last token, when the length is a multiple of 64, lands
  // on the first unit of the array after it, which the reverse scan writes
  // before anything reads it)
  float* s0_array = reinterpret_cast<float*>(ws + plan.ws_off) +
                    kda::bwd::dd_off(kda::bwd::S0M, plan.n_chunks * shape->num_heads, shape->d_k);
  f.snapshots = plan.n_snap <= 0 ? nullptr
                : plan.s0_in_place ? s0_array + (int64_t)shape->num_heads * shape->d_k * shape->d_k
                                   : reinterpret_cast<float*>(ws + plan.snap_off);
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
  f.one_seq = plan.fwd.one_seq;
  f.one_tok0 = plan.fwd.one_tok0;
  f.one_len = plan.fwd.one_len;
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
  b.states = plan.s0_in_place ? nullptr : reinterpret_cast<const float*>(ws + plan.snap_off);
  b.s0_in_place = plan.s0_in_place ? 1 : 0;
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
  return KDA_OK;
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
  *bytes = plan_full(shape, num_seqs, cu_seqlens_host, snapshot_interval, segment_tokens,
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
  int rc = validate_prefill(shape, num_seqs, cu_seqlens_host, cu_seqlens_dev, chunk, snapshot_interval,
                            segment_tokens, q, k, v, alpha, beta, initial_state, o, final_state, snapshots,
                            workspace, workspace_bytes);
  if (rc != KDA_OK) return rc;
  const int64_t T = cu_seqlens_host[num_seqs];
  const int64_t n_snap = snapshot_slots(num_seqs, cu_seqlens_host, snapshot_interval);
  const FullPlan plan = plan_full(shape, num_seqs, cu_seqlens_host, snapshot_interval, segment_tokens,
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

  const Geometry& geo = plan.geo;
  const hipStream_t st = static_cast<hipStream_t>(hip_stream);
  char* ws = static_cast<char*>(workspace);
  kda::PrefillArgs a{};
  a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.init = initial_state;
  a.o = o; a.final_state = final_state; a.snapshots = snaps_dev;
  hipError_t e = hipSuccess;
  const size_t H = (size_t)shape->num_heads, es = shape->qkv_dtype == KDA_BF16 ? 2 : 4;
  const int64_t dsz = geo.d, vrow = (int64_t)shape->d_v, half = (int64_t)shape->d_v * geo.d * 4;
  if (geo.pad) {
    // d_k = 2 d_v: values and states padded with zero rows in the workspace
    a.v = ws + plan.v_off;
    a.o = reinterpret_cast<float*>(ws + plan.o_off);
    a.final_state = reinterpret_cast<float*>(ws + plan.fin_off);
    a.snapshots = n_snap > 0 ? reinterpret_cast<float*>(ws + plan.snap_off) : nullptr;
    e = kda::launch_copy_rows(v, ws + plan.v_off, T * (int64_t)H, vrow * es, dsz * es, vrow * es, (dsz - vrow) * es, st);
    if (e == hipSuccess && initial_state) {
      a.init = reinterpret_cast<const float*>(ws + plan.init_off);
      e = kda::launch_copy_rows(initial_state, ws + plan.init_off, (int64_t)num_seqs * H, half, 2 * half, half,
                                half, st);
    }
    if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "prefill padding failed: %s", hipGetErrorString(e));
  }
  a.cu_dev = cu_seqlens_dev;
  a.num_seqs = num_seqs;
  a.H = geo.H;
  a.qk_shift = geo.qk_shift;
  a.interval = snapshot_interval;
  a.seg_chunks = plan.kern.seg_chunks;
  a.n_items = plan.kern.n_items;
  a.items = reinterpret_cast<kda::PrefillItem*>(ws + plan.kern.items_off);
  a.seq_first_item = reinterpret_cast<int32_t*>(ws + plan.kern.first_off);
  a.seg_maps = plan.kern.seg_chunks > 0 ? reinterpret_cast<float*>(ws + plan.kern.maps_off) : nullptr;
  a.seg_states = plan.kern.seg_chunks > 0 ? reinterpret_cast<float*>(ws + plan.kern.states_off) : nullptr;
  a.seg_wu = plan.kern.seg_chunks > 0 ? static_cast<void*>(ws + plan.kern.wu_off) : nullptr;
  a.any_whole = plan.kern.any_whole;
  a.one_seq = plan.kern.one_seq;
  a.one_tok0 = plan.kern.one_tok0;
  a.one_len = plan.kern.one_len;
  e = kda::launch_prefill(a, geo.d, shape->qkv_dtype == KDA_BF16, shape->gate == KDA_GATE_PER_KEY, st);
  if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "prefill launch failed: %s", hipGetErrorString(e));
  if (geo.pad) {
    e = kda::launch_copy_rows(a.o, o, T * (int64_t)H, dsz * 4, vrow * 4, vrow * 4, 0, st);
    if (e == hipSuccess)
      e = kda::launch_copy_rows(a.final_state, final_state, (int64_t)num_seqs * H, 2 * half, half, half, 0, st);
    if (e == hipSuccess && n_snap > 0)
      e = kda::launch_copy_rows(a.snapshots, snaps_dev, n_snap * (int64_t)H, 2 * half, half, half, 0, st);
    if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "prefill output copy failed: %s", hipGetErrorString(e));
  }
  g_err[0] = '\0';
  return KDA_OK;
}

int kda_prefill_chunked_noalloc(const kda_shape* shape, int32_t num_seqs,
                                const int64_t* cu_seqlens_host, const int64_t* cu_seqlens_dev,
                                int32_t chunk, int64_t snapshot_interval,
                                const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta, const float* initial_state,
                                float* o, float* final_state, float* snapshots, void* hip_stream) {
  // never segmented: the work table (one 40-byte item per sequence and the
  // first-item index) is all the scratch the kernels use
  int rc = validate_prefill(shape, num_seqs, cu_seqlens_host, cu_seqlens_dev, chunk, snapshot_interval, 0, q, k, v,
                            alpha, beta, initial_state, o, final_state, snapshots, nullptr, 0);
  if (rc != KDA_OK) return rc;
  const size_t need = plan_full(shape, num_seqs, cu_seqlens_host, snapshot_interval, 0, 0).bytes;
  if (need > kScratchBytes)
    return fail(KDA_ERR_WORKSPACE,
                "kda_prefill_chunked_noalloc: this call needs %zu bytes of scratch, the static scratch holds %zu "
                "(about 23000 sequences with d_v >= d_k; far fewer tokens with d_k = 2 d_v)",
                need, kScratchBytes);
  if (num_seqs == 0) {
    g_err[0] = '\0';
    return KDA_OK;
  }
  void* ws = scratch_address();
  if (!ws) return KDA_ERR_DEVICE;
  return kda_prefill_chunked(shape, num_seqs, cu_seqlens_host, cu_seqlens_dev, chunk, snapshot_interval, 0, q, k,
                             v, alpha, beta, initial_state, o, final_state, snapshots, ws, kScratchBytes,
                             hip_stream);
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
  {
    const size_t bh = (size_t)batch * shape->num_heads, es = shape->qkv_dtype == KDA_BF16 ? 2 : 4;
    const size_t a_n = bh * (shape->gate == KDA_GATE_PER_KEY ? (size_t)shape->d_k : 1) * sizeof(float);
    const Range ins[] = {{q, bh * shape->d_k * es, "q"}, {k, bh * shape->d_k * es, "k"},
                         {v, bh * shape->d_v * es, "v"}, {alpha, a_n, "alpha"}, {beta, bh * sizeof(float), "beta"},
                         {state, bh * shape->d_k * shape->d_v * sizeof(float), "state"}};
    rc = check_disjoint(Range{o, bh * shape->d_v * sizeof(float), "o"}, ins, 6);
    if (rc == KDA_OK) rc = check_disjoint(ins[5], ins, 5);
    if (rc != KDA_OK) return rc;
  }
  kda::DecodeArgs a{q, k, v, alpha, beta, state, o, batch, shape->num_heads};
  hipError_t e = kda::launch_decode(a, shape->d_k, shape->d_v, shape->qkv_dtype == KDA_BF16,
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
  {
    const size_t bh = (size_t)batch * shape->num_heads, bnh = bh * (size_t)n_tok;
    const size_t es = shape->qkv_dtype == KDA_BF16 ? 2 : 4, st = (size_t)shape->d_k * shape->d_v * sizeof(float);
    const size_t a_n = bnh * (shape->gate == KDA_GATE_PER_KEY ? (size_t)shape->d_k : 1) * sizeof(float);
    const Range ins[] = {{q, bnh * shape->d_k * es, "q"}, {k, bnh * shape->d_k * es, "k"},
                         {v, bnh * shape->d_v * es, "v"}, {alpha, a_n, "alpha"}, {beta, bnh * sizeof(float), "beta"},
                         {commit, (size_t)batch * sizeof(int32_t), "commit"}, {state, bh * st, "state"}};
    const Range ro{o, bnh * shape->d_v * sizeof(float), "o"}, rt{token_states, bnh * st, "token_states"};
    rc = check_disjoint(ro, ins, 7);
    if (rc == KDA_OK) rc = check_disjoint(rt, ins, 7);
    if (rc == KDA_OK) rc = check_disjoint(ins[6], ins, 6);
    if (rc == KDA_OK) rc = check_disjoint(ro, &rt, 1);
    if (rc != KDA_OK) return rc;
  }
  kda::DecodeArgs a{q, k, v, alpha, beta, state, o, batch, shape->num_heads, n_tok, token_states, commit};
  hipError_t e = kda::launch_decode_tokens(a, shape->d_k, shape->d_v, shape->qkv_dtype == KDA_BF16,
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
  int rc = check_shape(shape, true);
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

int kda_layer_prefill_workspace_size(const kda_shape* shape, int32_t num_seqs,
                                     const int64_t* cu_seqlens_host, int32_t chunk,
                                     int64_t snapshot_interval, int64_t segment_tokens, size_t* bytes) {
  if (!bytes) return fail(KDA_ERR_ARG, "bytes is NULL");
  int rc = check_shape(shape, true);
  if (rc != KDA_OK) return rc;
  rc = check_prefill_args(shape, num_seqs, cu_seqlens_host, chunk, snapshot_interval, segment_tokens);
  if (rc != KDA_OK) return rc;
  *bytes = plan_layer(shape, num_seqs, cu_seqlens_host, snapshot_interval, segment_tokens,
                      segment_tokens < 0 ? device_cu_count() : 0).bytes;
  g_err[0] = '\0';
  return KDA_OK;
}

int kda_layer_prefill(const kda_shape* shape, int32_t num_seqs,
                      const int64_t* cu_seqlens_host, const int64_t* cu_seqlens_dev,
                      int32_t chunk, int64_t snapshot_interval, int64_t segment_tokens,
                      const void* q, const void* k, const void* v,
                      const float* alpha, const float* beta, const float* initial_state,
                      const void* g_logit, const float* norm_w, float eps, int32_t out_dtype,
                      void* out, float* final_state, float* snapshots,
                      void* workspace, size_t workspace_bytes, void* hip_stream) {
  int rc = check_shape(shape, true);
  if (rc != KDA_OK) return rc;
  if (out_dtype != KDA_BF16 && out_dtype != KDA_F32)
    return fail(KDA_ERR_ARG, "out_dtype must be KDA_BF16 or KDA_F32 (got %d)", out_dtype);
  if (!(eps >= 0.f)) return fail(KDA_ERR_ARG, "eps must be >= 0");
  const size_t out_es = out_dtype == KDA_BF16 ? 2 : 4;
  rc = validate_prefill(shape, num_seqs, cu_seqlens_host, cu_seqlens_dev, chunk, snapshot_interval, segment_tokens,
                        q, k, v, alpha, beta, initial_state, out, final_state, snapshots, workspace, workspace_bytes,
                        out_es, "out");
  if (rc != KDA_OK) return rc;
  const int64_t T = cu_seqlens_host[num_seqs];
  const int64_t n_snap = snapshot_slots(num_seqs, cu_seqlens_host, snapshot_interval);
  const size_t H = (size_t)shape->num_heads, d = (size_t)shape->d_v, es = shape->qkv_dtype == KDA_BF16 ? 2 : 4;
  if (T > 0) {
    if (!g_logit || !norm_w) return fail(KDA_ERR_ARG, "g_logit and norm_w must be non-NULL when T > 0");
    const PtrReq reqs[] = {{g_logit, 16, "g_logit"}, {norm_w, 16, "norm_w"}};
    rc = check_align(reqs, 2);
    if (rc != KDA_OK) return rc;
    const size_t st = d * d * sizeof(float);
    const Range ins[] = {{g_logit, (size_t)T * H * d * es, "g_logit"}, {norm_w, d * sizeof(float), "norm_w"}};
    const Range outs[] = {{out, (size_t)T * H * d * out_es, "out"}, {final_state, (size_t)num_seqs * H * st, "final_state"},
                          {n_snap > 0 ? snapshots : nullptr, (size_t)n_snap * H * st, "snapshots"}};
    for (const Range& o : outs)
      if ((rc = check_disjoint(o, ins, 2)) != KDA_OK) return rc;
  }
  const LayerPlan plan = plan_layer(shape, num_seqs, cu_seqlens_host, snapshot_interval, segment_tokens,
                                    segment_tokens < 0 ? device_cu_count() : 0);
  if (num_seqs > 0 && (!workspace || workspace_bytes < plan.bytes))
    return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", plan.bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (num_seqs == 0) {
    g_err[0] = '\0';
    return KDA_OK;
  }
  char* ws = static_cast<char*>(workspace);
  const hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (!plan.fused) {
    // the recurrence into an fp32 o in the workspace, then the back-end kernel
    float* o = reinterpret_cast<float*>(ws + plan.aux_off);
    rc = kda_prefill_chunked(shape, num_seqs, cu_seqlens_host, cu_seqlens_dev, chunk, snapshot_interval,
                             segment_tokens, q, k, v, alpha, beta, initial_state, o, final_state, snapshots,
                             workspace, plan.aux_off, hip_stream);
    if (rc != KDA_OK) return rc;
    kda::LayerBackArgs b{o, g_logit, norm_w, out, eps, T * (int64_t)H, shape->qkv_dtype == KDA_BF16};
    const hipError_t e = kda::launch_layer_back(b, (int)d, out_dtype == KDA_BF16, st);
    if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "layer back launch failed: %s", hipGetErrorString(e));
    g_err[0] = '\0';
    return KDA_OK;
  }
  float* snaps_dev = nullptr;
  if (n_snap > 0) {
    rc = resolve_snapshots(snapshots, &snaps_dev);
    if (rc != KDA_OK) return rc;
  }
  const PrefillPlan& kp = plan.pre.kern;
  kda::PrefillArgs a{};
  a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.init = initial_state;
  a.o = nullptr; a.final_state = final_state; a.snapshots = snaps_dev;
  a.cu_dev = cu_seqlens_dev;
  a.num_seqs = num_seqs;
  a.H = shape->num_heads;
  a.qk_shift = 0;
  a.interval = snapshot_interval;
  a.seg_chunks = kp.seg_chunks;
  a.n_items = kp.n_items;
  a.items = reinterpret_cast<kda::PrefillItem*>(ws + kp.items_off);
  a.seq_first_item = reinterpret_cast<int32_t*>(ws + kp.first_off);
  a.seg_maps = reinterpret_cast<float*>(ws + kp.maps_off);
  a.seg_states = reinterpret_cast<float*>(ws + kp.states_off);
  a.seg_wu = static_cast<void*>(ws + kp.wu_off);
  a.any_whole = kp.any_whole;
  a.one_seq = kp.one_seq;
  a.one_tok0 = kp.one_tok0;
  a.one_len = kp.one_len;
  a.g_logit = g_logit;
  a.norm_w = norm_w;
  a.out = out;
  a.out_sink = ws + plan.aux_off;
  a.eps = eps;
  a.out_bf16 = out_dtype == KDA_BF16;
  const hipError_t e = kda::launch_prefill(a, (int)d, true, shape->gate == KDA_GATE_PER_KEY, st);
  if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "layer prefill launch failed: %s", hipGetErrorString(e));
  g_err[0] = '\0';
  return KDA_OK;
}

int kda_prefill_backward_workspace_size(const kda_shape* shape, int32_t num_seqs,
                                        const int64_t* cu_seqlens_host, size_t* bytes) {
  if (!bytes) return fail(KDA_ERR_ARG, "bytes is NULL");
  int rc = check_shape(shape, true);
  if (rc != KDA_OK) return rc;
  rc = check_cu(num_seqs, cu_seqlens_host);
  if (rc != KDA_OK) return rc;
  *bytes = plan_backward_grouped(shape, num_seqs, cu_seqlens_host, device_cu_count()).bytes;
  g_err[0] = '\0';
  return KDA_OK;
}

int kda_prefill_backward(const kda_shape* shape, int32_t num_seqs, const int64_t* cu_seqlens_host,
                         const int64_t* cu_seqlens_dev, const void* q, const void* k, const void* v,
                         const float* alpha, const float* beta, const float* initial_state, const float* d_o,
                         const float* d_final_state, float* dq, float* dk, float* dv, float* dalpha,
                         float* dbeta, float* d_initial_state, void* workspace, size_t workspace_bytes,
                         void* hip_stream) {
  int rc = check_shape(shape, true);
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
  {
    // every gradient is written while the inputs are read: no output may
    // overlap an input or another output, except d_initial_state = d_final_state
    const size_t H = (size_t)shape->num_heads, d = (size_t)shape->d_k, es = shape->qkv_dtype == KDA_BF16 ? 2 : 4;
    const size_t tokh = (size_t)T * H, st = (size_t)num_seqs * H * d * d * sizeof(float);
    const size_t a_n = tokh * (shape->gate == KDA_GATE_PER_KEY ? d : 1) * sizeof(float);
    const Range ins[] = {{q, tokh * d * es, "q"}, {k, tokh * d * es, "k"}, {v, tokh * d * es, "v"},
                         {alpha, a_n, "alpha"}, {beta, tokh * sizeof(float), "beta"},
                         {initial_state, st, "initial_state"}, {d_o, tokh * d * sizeof(float), "d_o"},
                         {cu_seqlens_dev, ((size_t)num_seqs + 1) * sizeof(int64_t), "cu_seqlens_dev"},
                         {workspace, workspace_bytes, "workspace"}, {d_final_state, st, "d_final_state"}};
    const Range outs[] = {{dq, tokh * d * sizeof(float), "dq"}, {dk, tokh * d * sizeof(float), "dk"},
                          {dv, tokh * d * sizeof(float), "dv"}, {dalpha, a_n, "dalpha"},
                          {dbeta, tokh * sizeof(float), "dbeta"}, {d_initial_state, st, "d_initial_state"}};
    for (int i = 0; i < 6 && rc == KDA_OK; ++i) {
      const bool same = i == 5 && d_initial_state == d_final_state;
      rc = check_disjoint(outs[i], ins, same ? 9 : 10);
      if (rc == KDA_OK && i + 1 < 6) rc = check_disjoint(outs[i], outs + i + 1, 5 - i);
    }
    if (rc != KDA_OK) return rc;
  }
  if (num_seqs == 0) {
    g_err[0] = '\0';
    return KDA_OK;
  }
  const GroupedBackward gp = plan_backward_grouped(shape, num_seqs, cu_seqlens_host, device_cu_count());
  if (!workspace || workspace_bytes < gp.bytes)
    return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", gp.bytes,
                workspace ? workspace_bytes : (size_t)0);
  char* ws = static_cast<char*>(workspace);
  const hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (gp.groups == 1) {
    rc = run_backward(shape, num_seqs, cu_seqlens_dev, gp.plan, q, k, v, alpha, beta, initial_state, d_o,
                      d_final_state, dq, dk, dv, dalpha, dbeta, d_initial_state, ws, st);
    if (rc != KDA_OK) return rc;
    g_err[0] = '\0';
    return KDA_OK;
  }
  // heads in groups: gather, run, scatter (row copies over tokens or sequences)
  const int H = shape->num_heads;
  const int64_t N = num_seqs, d = shape->d_k;
  const int64_t es = shape->qkv_dtype == KDA_BF16 ? 2 : 4;
  const int64_t a_el = shape->gate == KDA_GATE_PER_KEY ? d : 1, dd4 = d * d * 4;
  for (int h0 = 0; h0 < H; h0 += gp.Hg) {
    const int hg = H - h0 < gp.Hg ? H - h0 : gp.Hg;
    kda_shape gs = *shape;
    gs.num_heads = hg;
    const BackwardPlan plan = plan_backward(&gs, num_seqs, cu_seqlens_host, device_cu_count());
    auto at = [&](size_t off) { return ws + off; };
    // gather: rows of T tokens (or N sequences), this group's heads
    auto gather = [&](const void* src, size_t dst_off, int64_t rows, int64_t head_bytes) {
      return kda::launch_copy_rows(static_cast<const char*>(src) + h0 * head_bytes, at(dst_off), rows, H * head_bytes,
                                   hg * head_bytes, hg * head_bytes, 0, st);
    };
    auto scatter = [&](size_t src_off, void* dst, int64_t rows, int64_t head_bytes) {
      return kda::launch_copy_rows(at(src_off), static_cast<char*>(dst) + h0 * head_bytes, rows, hg * head_bytes,
                                   H * head_bytes, hg * head_bytes, 0, st);
    };
    hipError_t e = gather(q, gp.q_off, T, d * es);
    if (e == hipSuccess) e = gather(k, gp.k_off, T, d * es);
    if (e == hipSuccess) e = gather(v, gp.v_off, T, d * es);
    if (e == hipSuccess) e = gather(alpha, gp.a_off, T, a_el * 4);
    if (e == hipSuccess) e = gather(beta, gp.b_off, T, 4);
    if (e == hipSuccess) e = gather(d_o, gp.do_off, T, d * 4);
    if (e == hipSuccess && initial_state) e = gather(initial_state, gp.init_off, N, dd4);
    if (e == hipSuccess && d_final_state) e = gather(d_final_state, gp.df_off, N, dd4);
    if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "backward gather failed: %s", hipGetErrorString(e));
    rc = run_backward(&gs, num_seqs, cu_seqlens_dev, plan, at(gp.q_off), at(gp.k_off), at(gp.v_off),
                      reinterpret_cast<const float*>(at(gp.a_off)), reinterpret_cast<const float*>(at(gp.b_off)),
                      initial_state ? reinterpret_cast<const float*>(at(gp.init_off)) : nullptr,
                      reinterpret_cast<const float*>(at(gp.do_off)),
                      d_final_state ? reinterpret_cast<const float*>(at(gp.df_off)) : nullptr,
                      reinterpret_cast<float*>(at(gp.dq_off)), reinterpret_cast<float*>(at(gp.dk_off)),
                      reinterpret_cast<float*>(at(gp.dv_off)), reinterpret_cast<float*>(at(gp.da_off)),
                      reinterpret_cast<float*>(at(gp.db_off)),
                      d_initial_state ? reinterpret_cast<float*>(at(gp.di_off)) : nullptr, ws, st);
    if (rc != KDA_OK) return rc;
    e = scatter(gp.dq_off, dq, T, d * 4);
    if (e == hipSuccess) e = scatter(gp.dk_off, dk, T, d * 4);
    if (e == hipSuccess) e = scatter(gp.dv_off, dv, T, d * 4);
    if (e == hipSuccess) e = scatter(gp.da_off, dalpha, T, a_el * 4);
    if (e == hipSuccess) e = scatter(gp.db_off, dbeta, T, 4);
    if (e == hipSuccess && d_initial_state) e = scatter(gp.di_off, d_initial_state, N, dd4);
    if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "backward scatter failed: %s", hipGetErrorString(e));
  }
  g_err[0] = '\0';
  return KDA_OK;
}

}  // extern "C"
