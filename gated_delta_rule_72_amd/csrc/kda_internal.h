// kda_internal.h — shared definitions of the gfx950 kernels and the host API
// of libkda.so (not part of the public ABI; see include/kda.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// bf16 bit pattern -> fp32 (exact: bf16 is the upper half of an fp32).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// sigmoid with the hardware reciprocal (1 ulp) instead of an IEEE divide (the
// layer's gates and output gate; the prefill's fused back end uses the same one,
// so fused and separate back ends give the same bits)
__device__ __forceinline__ float sigmoid_rcp(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Four consecutive q/k/v elements starting at element index `idx`.
template <bool BF16>
__device__ __forceinline__ f32x4 load4(const void* base, int64_t idx) {
  if constexpr (BF16) {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + idx);
    f32x4 r;
    r[0] = bf16_bits_to_f32(w.x & 0xFFFFu);
    r[1] = bf16_bits_to_f32(w.x >> 16);
    r[2] = bf16_bits_to_f32(w.y & 0xFFFFu);
    r[3] = bf16_bits_to_f32(w.y >> 16);
    return r;
  } else {
    return *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx);
  }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* base, int64_t idx) {
  if constexpr (BF16)
    return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[idx]);
  else
    return static_cast<const float*>(base)[idx];
}

// ---- launch entry points (defined in the .hip files) -----------------------

struct DecodeArgs {
  const void *q, *k, *v;
  const float *alpha, *beta;
  float *state, *o;
  int32_t batch, H;
  int32_t n_tok;             // tokens per sequence (multi-token path)
  float* token_states;       // [batch, n_tok, H, dv, dk] or null
  const int32_t* commit;     // [batch] tokens to commit to `state`, or null (all)
};
hipError_t launch_decode(const DecodeArgs& a, int dk, int dv, bool bf16, bool per_key, hipStream_t s);
hipError_t launch_decode_tokens(const DecodeArgs& a, int dk, int dv, bool bf16, bool per_key, hipStream_t s);

// One unit of prefill work: a contiguous run of chunks of one sequence (the
// whole sequence, or one segment of it).
struct PrefillItem {
  int64_t tok_begin;   // first token (global index into q/k/v/o)
  int64_t tok_in_seq;  // position of tok_begin inside its sequence
  int64_t snap_base;   // first snapshot slot of the sequence
  int32_t n_tokens;    // tokens in this item
  int32_t seq;         // sequence index n
  int32_t seg;         // segment index within the sequence (0 if unsegmented)
  int32_t n_segs;      // segments of this sequence
};

struct PrefillArgs {
  const void *q, *k, *v;
  const float *alpha, *beta;
  const float* init;         // [N,H,dv,dk] or null
  float *o, *final_state, *snapshots;
  const int64_t* cu_dev;     // [N+1]
  int32_t num_seqs, H;
  int64_t interval;          // snapshot interval (0 = none)
  int32_t seg_chunks;        // chunks per segment (0 = unsegmented)
  int32_t n_items;           // work items (sequences or sequence segments)
  PrefillItem* items;        // workspace: [n_items]
  int32_t* seq_first_item;   // workspace: [N] first item of each sequence (segmented)
  float* seg_maps;           // workspace: per (item, head) M (dk x dk) then N (dv x dk)
  float* seg_states;         // workspace: per (item, head) start state (dv x dk)
  void* seg_wu;              // workspace: per (item, head, chunk) the chunk's W (fp16, the
                             // LDS layout the map pass leaves it in) and U' (fp32, one
                             // accumulator tile per lane), reused by pass 3
  int32_t any_whole;         // segmented plan: some sequence is not split (needs its own pass)
  // One sequence (num_seqs = 1): the kernels form each work item from its
  // first token and length (segments of seg_chunks chunks, or the whole
  // sequence) and no work table is built
  int32_t one_seq;
  int64_t one_tok0, one_len;
  int32_t qk_shift;          // 0, or 1 when d_v = 2 d_k: H counts value heads of d_k state rows,
                             // and value head h takes q, k, alpha, beta of head h >> 1 of H / 2
  // Layer back end fused into pass 3 (scalar gate, bf16, d = 128, every
  // sequence split): when `out` is set, pass 3 writes
  // out = o * rsqrt(mean over d of o^2 + eps) * norm_w * sigmoid(g_logit)
  // ([T, H, d], bf16 or fp32 as out_bf16) instead of o
  const void* g_logit;       // [T, H, d] bf16
  const float* norm_w;       // [d]
  void* out;
  void* out_sink;            // 16 bytes of workspace: stores of rows past a chunk's end land
                             // there (their values are discarded)
  float eps;
  int32_t out_bf16;
};
hipError_t launch_prefill(PrefillArgs a, int d, bool bf16, bool per_key, hipStream_t s);
// Row copy with zero fill: for r < n_rows, bytes [0, copy) of dst row r
// (stride dst_stride) take those of src row r (stride src_stride) and bytes
// [copy, copy + fill) are zeroed. Sizes, strides and both pointers are
// multiples of 4 bytes (moved in 16-byte pieces when all are multiples of 16).
hipError_t launch_copy_rows(const void* src, void* dst, int64_t n_rows, int64_t src_stride,
                            int64_t dst_stride, int64_t copy, int64_t fill, hipStream_t s);
// Bytes of one chunk's stored W and U' at d = d_k = d_v: W as 64 rows of d + 8
// fp16 (the LDS row stride, a whole number of KiB), then U' as 64 x d fp32.
constexpr size_t wu_w_bytes(int d) { return (size_t)64 * (d + 8) * 2; }
constexpr size_t wu_chunk_bytes(int d) { return wu_w_bytes(d) + (size_t)64 * d * 4; }

// Layer front end: conv-4 + SiLU (+ L2 norm for q, k), gates, carried conv state.
struct LayerFrontArgs {
  const void *xq, *xk, *xv;         // [T, H, d] conv inputs (qkv dtype)
  const float* conv_w;              // [3, H, d, 4] taps, oldest first
  const void* conv_state_in;        // [N, 3, 3, H, d] (qkv dtype) or null
  const float *alpha_logit, *beta_logit;
  float alpha_bias;
  void *q, *k, *v;                  // [T, H, d] outputs (qkv dtype)
  float *alpha, *beta;
  void* conv_state_out;             // [N, 3, 3, H, d] or null
  const int64_t* cu;                // device cu_seqlens [N+1]
  int32_t num_seqs, H;
  int64_t T;
};
hipError_t launch_layer_front(const LayerFrontArgs& a, int d, bool bf16, bool per_key, hipStream_t s);

// Layer back end: RMSNorm over d_v times a sigmoid output gate.
struct LayerBackArgs {
  const float* o;
  const void* g_logit;              // fp32, or bf16 when g_bf16
  const float* norm_w;
  void* out;
  float eps;
  int64_t rows;                     // T * H
  int32_t g_bf16;
};
hipError_t launch_layer_back(const LayerBackArgs& a, int d, bool out_bf16, hipStream_t s);

// Backward pass of the chunked prefill (gradients of the token recurrence).
// Per (chunk, head) unit b = chunk * H + h, the workspace holds fp32 arrays of
// 64 x D (chunk rows x channels), 64 x 64 and D x D, each as one region of
// n_units consecutive blocks, followed by exp(Gamma_n) [D] and beta [64].
namespace bwd {
enum ArrND { KP, KM, QP, XA, QA, KT, YB, DOF, XP, WM, UM, ZU, DQP, DQA, DKM, DKT, DW, DX, DY, DKP, GG, N_ND };
enum ArrNN { PM, AM, BM, DBM, DAM, TM, DLM, N_NN };
enum ArrDD { S0M, DSN, EM, N_DD };
__host__ __device__ constexpr int64_t nd_off(int a, int64_t units, int d) { return (int64_t)a * units * 64 * d; }
__host__ __device__ constexpr int64_t nn_off(int a, int64_t units, int d) {
  return nd_off(N_ND, units, d) + (int64_t)a * units * 64 * 64;
}
__host__ __device__ constexpr int64_t dd_off(int a, int64_t units, int d) {
  return nn_off(N_NN, units, d) + (int64_t)a * units * d * d;
}
__host__ __device__ constexpr int64_t egn_off(int64_t units, int d) { return dd_off(N_DD, units, d); }
__host__ __device__ constexpr int64_t beta_off(int64_t units, int d) { return egn_off(units, d) + units * d; }
__host__ __device__ constexpr int64_t floats(int64_t units, int d) { return beta_off(units, d) + units * 64; }
}  // namespace bwd

struct BackwardArgs {
  const void *q, *k, *v;
  const float *alpha, *beta;
  const float* init;         // [N,H,dv,dk] or null
  const float* d_o;          // [T,H,dv]
  const float* d_final;      // [N,H,dv,dk] or null
  float *dq, *dk, *dv, *dalpha, *dbeta;
  float* d_init;             // [N,H,dv,dk] or null
  const int64_t* cu_dev;     // [N+1]
  int32_t num_seqs, H;
  int64_t n_chunks;          // chunks over all sequences
  const float* states;       // forward states after every 64 tokens, snapshot slot order
  int32_t s0_in_place;       // one sequence: the forward wrote those states straight into
                             // the chunk-start array (ws, S0M from its unit H on), so only a
                             // sequence's first chunk takes its start state from init
  int64_t* chunk_base;       // workspace [N+1]: first chunk of each sequence
  int64_t* snap_base;        // workspace [N+1]: first 64-token state slot of each sequence
  int64_t* item_base;        // workspace [N+1]: first scan segment of each sequence
  int32_t seg_chunks;        // chunks per scan segment (0: one segment per sequence)
  int64_t n_items;           // scan segments over all sequences (at least one per sequence)
  float* seg_maps;           // workspace [n_items, H, 2, d, d]: each segment's map (M, then N)
  float* seg_end;            // workspace [n_items, H, d, d]: dS^T at each segment's end
  float* ws;                 // workspace: bwd::floats(n_chunks * H, d) fp32
};
hipError_t launch_backward(const BackwardArgs& a, int d, bool bf16, bool per_key, hipStream_t s);

}  // namespace kda
