// kda_decode.hip — one O(1)-state decode step of the gated delta rule.
//
// Page "Modele hybrydowe: co Gated DeltaNet zastępuje w cache KV" (trefon.com),
// section "Gated DeltaNet: dodaj zanik" (update) and "Atencja liniowa: stan o
// stałym rozmiarze" (read-out o_t = S_t q_t). Row i of the d_v x d_k state is
// updated on its own:
//     s' = s_i * a          (decay on the key axis; scalar gate: a = alpha)
//     p  = s' . k           (what the state predicts for k)
//     r  = s' . q
//     u  = beta (v_i - p)   (the written error)
//     s_i <- s' + u k
//     o_i = s_i . q = r + u (k . q)
// The step reads and writes each state element exactly once; the kernel is
// bound by HBM bandwidth (about 0.86 flop per byte).
//
// Several tokens per sequence (kda_decode_tokens: a speculative draft) run the
// same step in a loop with the state held in registers; the state after each
// token can be written out (rollback points, same page, section "Co stan
// rekurencyjny zmienia przy serwowaniu", item 2) and the state after a chosen
// prefix goes back to HBM.
//
// Mapping (d_k = DK, d_v = DV, each 64 or 128): one workgroup per (sequence,
// head), DV/32 wavefronts, 32 state rows per wavefront. A row is DK/4 lanes
// wide (one 16-byte float4 per lane), so a wavefront holds G = 256/DK rows side
// by side and every load instruction moves G consecutive rows (1 KiB). Each lane group
// keeps R = 32/G rows in registers and finishes all 2R dot products of its
// rows with one butterfly reduce-scatter: log2(DK/4) shuffle steps in which
// the number of live partial sums halves, leaving lane j of the group with
// the full sum of value j.
#include "kda_internal.h"

namespace kda {
namespace {

// x from lane (lane ^ M), M < 32: quad permutes (DPP) for M = 1, 2, the
// swizzle crossbar in xor mode for larger M; neither touches LDS memory.
template <int M>
__device__ __forceinline__ float xor_lane(float x) {
  const int xi = __float_as_int(x);
  int r;
  if constexpr (M == 1)
    r = __builtin_amdgcn_update_dpp(xi, xi, 0xB1, 0xF, 0xF, false);      // quad_perm [1,0,3,2]
  else if constexpr (M == 2)
    r = __builtin_amdgcn_update_dpp(xi, xi, 0x4E, 0xF, 0xF, false);      // quad_perm [2,3,0,1]
  else
    r = __builtin_amdgcn_ds_swizzle(xi, 0x1F | (M << 10));               // bit mode: lane ^ M
  return __int_as_float(r);
}

// Lanes [base, base+N) of a group hold vals[0..N) each; afterwards lane
// base+j returns the sum over the group of vals[j].
template <int N, int M>
__device__ __forceinline__ void reduce_scatter_step(float (&vals)[N], int lane_in_group) {
  const bool upper = (lane_in_group & M) != 0;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    const float send = upper ? vals[j] : vals[j + M];
    const float keep = upper ? vals[j + M] : vals[j];
    vals[j] = keep + xor_lane<M>(send);
  }
}
template <int N>
__device__ __forceinline__ float reduce_scatter(float (&vals)[N], int lane_in_group) {
  if constexpr (N >= 32) reduce_scatter_step<N, 16>(vals, lane_in_group);
  if constexpr (N >= 16) reduce_scatter_step<N, 8>(vals, lane_in_group);
  if constexpr (N >= 8) reduce_scatter_step<N, 4>(vals, lane_in_group);
  if constexpr (N >= 4) reduce_scatter_step<N, 2>(vals, lane_in_group);
  reduce_scatter_step<N, 1>(vals, lane_in_group);
  return vals[0];
}

template <int N>
__device__ __forceinline__ float group_allreduce(float x) {
  if constexpr (N >= 32) x += xor_lane<16>(x);
  if constexpr (N >= 16) x += xor_lane<8>(x);
  x += xor_lane<4>(x);
  x += xor_lane<2>(x);
  x += xor_lane<1>(x);
  return x;
}

// MULTI: n_tok tokens per sequence ([batch, n_tok, H, d] inputs), the state
// kept in registers between them; the state after token t goes to
// token_states (KEEP: token_states given) and, for t + 1 == commit, back to
// `state`. KEEP is a template flag so that the per-token stores are not under
// a branch: with them under one, the wait for the next token's inputs would
// also wait for the stores.
template <int DK, int DV, bool BF16, bool PER_KEY, bool MULTI, bool KEEP>
__global__ __launch_bounds__(DV * 2) __attribute__((amdgpu_waves_per_eu(1, KEEP ? 2 : 8)))
void decode_kernel(DecodeArgs a) {
  constexpr int LPR = DK / 4;     // lanes per state row
  constexpr int G = 64 / LPR;     // rows side by side in a wavefront
  constexpr int R = 32 / G;       // rows per lane group
  static_assert(2 * R == LPR, "one reduced value per lane");

  const int bh = blockIdx.x;      // (sequence, head) = b * H + h
  const int b = bh / a.H, h = bh % a.H;
  const int wave = threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  const int g = lane / LPR;       // lane group within the wavefront
  const int li = lane % LPR;      // lane within the group; owns columns 4li..4li+3

  // rows of this lane group: wave*32 + r*G + g, r = 0..R-1
  float* state = a.state + (int64_t)bh * DV * DK;
  f32x4 s[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = wave * 32 + r * G + g;
    s[r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(state + (int64_t)row * DK + 4 * li));
  }

  const int n_tok = MULTI ? a.n_tok : 1;
  int commit = n_tok;
  if (MULTI && a.commit) commit = min(max(a.commit[b], 0), n_tok);

  // this lane's value row (lanes with even li use it)
  const int my_r = li >> 1;
  const int my_row = wave * 32 + my_r * G + g;
  struct TokenIn {
    f32x4 k, q, a;
    float beta, v;
  };
  // a token's inputs; the next token's are fetched while the current one runs
  auto load_token = [&](int t) {
    const int64_t tok = MULTI ? ((int64_t)b * n_tok + t) * a.H + h : bh;   // (sequence, token, head)
    const int64_t k_off = tok * DK;
    TokenIn x;
    x.k = load4<BF16>(a.k, k_off + 4 * li);
    x.q = load4<BF16>(a.q, k_off + 4 * li);
    if constexpr (PER_KEY) {
      x.a = *reinterpret_cast<const f32x4*>(a.alpha + k_off + 4 * li);
    } else {
      const float al = a.alpha[tok];
      x.a = f32x4{al, al, al, al};
    }
    x.beta = a.beta[tok];
    x.v = load1<BF16>(a.v, tok * DV + my_row);
    return x;
  };
  TokenIn next = load_token(0);

  // this lane's element offset in the state, re-derived from an opaque copy
  // of the thread index where it is used: hoisted out of the token loop, the
  // addresses of the R rows would hold 2R registers for the whole call
  auto lane_elem = [&]() __attribute__((always_inline)) {
    int tid = threadIdx.x;
    if constexpr (MULTI) asm volatile("" : "+v"(tid));
    return (wave * 32 + (tid % 64) / LPR) * DK + 4 * (tid % LPR);
  };
  auto step = [&](int t) __attribute__((always_inline)) {
    const int64_t tok = MULTI ? ((int64_t)b * n_tok + t) * a.H + h : bh;   // (sequence, token, head)
    const int64_t v_off = tok * DV;
    const TokenIn cur = next;
    // unconditional (the last token fetches itself again): a load under a
    // branch leaves the wait counts path-dependent, and the compiler then
    // waits for this token's stores before the next token starts
    if constexpr (MULTI) next = load_token(min(t + 1, n_tok - 1));
    const f32x4 kv = cur.k, qv = cur.q, av = cur.a;
    const float beta = cur.beta;

    float kq = kv[0] * qv[0] + kv[1] * qv[1] + kv[2] * qv[2] + kv[3] * qv[3];
    kq = group_allreduce<LPR>(kq);

    float vals[2 * R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      s[r] = s[r] * av;
      vals[2 * r] = s[r][0] * kv[0] + s[r][1] * kv[1] + s[r][2] * kv[2] + s[r][3] * kv[3];
      vals[2 * r + 1] = s[r][0] * qv[0] + s[r][1] * qv[1] + s[r][2] * qv[2] + s[r][3] * qv[3];
    }
    // lane li = 2r holds p_r, lane li = 2r+1 holds (s'_r . q)
    const float red = reduce_scatter<2 * R>(vals, li);
    float u = 0.f;
    if ((li & 1) == 0) u = beta * (cur.v - red);
    const float u_pair = xor_lane<1>(u);
    if constexpr (MULTI) {
      // o of the pair's row: the odd lane holds s'.q, the even lane u; both
      // lanes form the same sum from the same operands and store the same
      // bits to the same address, so no branch skips the even lanes' store
      const float r_pair = xor_lane<1>(red);
      a.o[v_off + my_row] = (li & 1) ? red + u_pair * kq : r_pair + u * kq;
    } else {
      if (li & 1) a.o[v_off + my_row] = red + u_pair * kq;
    }

    // u of row r sits in lane 2r of each lane group: read it wave-wide and keep
    // the copy of this lane's group
    float* snap = KEEP ? a.token_states + tok * DV * DK : nullptr;
    const int elem = MULTI ? lane_elem() : 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float ur = 0.f;
#pragma unroll
      for (int gg = 0; gg < G; ++gg) {
        const float x = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(u), gg * LPR + 2 * r));
        if (g == gg) ur = x;
      }
      s[r] = s[r] + ur * kv;
      if constexpr (KEEP)
        __builtin_nontemporal_store(s[r], reinterpret_cast<f32x4*>(snap + elem + r * G * DK));   // row wave*32 + r*G + g
      if constexpr (!MULTI) {
        const int row = wave * 32 + r * G + g;
        __builtin_nontemporal_store(s[r], reinterpret_cast<f32x4*>(state + (int64_t)row * DK + 4 * li));
      }
    }
  };
  if constexpr (!MULTI) {
    step(0);
  } else {
    // The tokens up to the commit point, the committed state, then the rest:
    // a store under a per-token test would leave the wait counts
    // path-dependent.
    for (int t = 0; t < commit; ++t) step(t);
    if (commit > 0) {
      const int elem = lane_elem();
#pragma unroll
      for (int r = 0; r < R; ++r)
        __builtin_nontemporal_store(s[r], reinterpret_cast<f32x4*>(state + elem + r * G * DK));
    }
    for (int t = commit; t < n_tok; ++t) step(t);
  }
}

template <int DK, int DV, bool BF16, bool PK, bool MULTI>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
  if (MULTI && a.token_states)
    hipLaunchKernelGGL((decode_kernel<DK, DV, BF16, PK, MULTI, MULTI>), dim3(a.batch * a.H), dim3(DV * 2), 0, s, a);
  else
    hipLaunchKernelGGL((decode_kernel<DK, DV, BF16, PK, MULTI, false>), dim3(a.batch * a.H), dim3(DV * 2), 0, s, a);
  return hipGetLastError();
}

template <int DK, int DV, bool MULTI>
hipError_t launch_dt(const DecodeArgs& a, bool bf16, bool per_key, hipStream_t s) {
  if (bf16) return per_key ? launch_t<DK, DV, true, true, MULTI>(a, s) : launch_t<DK, DV, true, false, MULTI>(a, s);
  return per_key ? launch_t<DK, DV, false, true, MULTI>(a, s) : launch_t<DK, DV, false, false, MULTI>(a, s);
}

template <bool MULTI>
hipError_t launch_any(const DecodeArgs& a, int dk, int dv, bool bf16, bool per_key, hipStream_t s) {
  if (dk == 64) return dv == 64 ? launch_dt<64, 64, MULTI>(a, bf16, per_key, s) : launch_dt<64, 128, MULTI>(a, bf16, per_key, s);
  return dv == 64 ? launch_dt<128, 64, MULTI>(a, bf16, per_key, s) : launch_dt<128, 128, MULTI>(a, bf16, per_key, s);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int dk, int dv, bool bf16, bool per_key, hipStream_t s) {
  return launch_any<false>(a, dk, dv, bf16, per_key, s);
}

hipError_t launch_decode_tokens(const DecodeArgs& a, int dk, int dv, bool bf16, bool per_key, hipStream_t s) {
  return launch_any<true>(a, dk, dv, bf16, per_key, s);
}

}  // namespace kda
