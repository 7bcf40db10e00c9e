// kda_backward.hip — backward pass of the chunked prefill on gfx950.
//
// Gradients of the loss sum_t <dO_t, o_t> + sum_n <dS_n, S_final,n> with
// respect to q, k, v, the gate, beta and the initial state, for the update of
// page "Modele hybrydowe: co Gated DeltaNet zastępuje w cache KV"
// (trefon.com), section "Gated DeltaNet: dodaj zanik", in the chunked form the
// forward uses (closing paragraph of "Co stan rekurencyjny zmienia przy
// serwowaniu": inside a chunk everything is a dense product; only chunk to
// chunk is sequential). With Gamma the in-chunk cumulative natural-log decay,
// a reference row c (row 31, or the last row of a shorter chunk: it cancels
// in every product and keeps each factor inside fp32), and per chunk
//   Kp = K e^(G-G_c), Km = K e^(G_c-G), Qp = Q e^(G-G_c), Ka = K e^G,
//   Qa = Q e^G, Kt = K e^(G_n-G), P = Kp Km^T, A = (I + strict_lower(B P))^-1,
//   X = B Ka, Y = B V, W = A X, U = A Y - W S0^T, Bm = lower(Qp Km^T)
// (B = Diag(beta)), the forward is O = Qa S0^T + Bm U and
// S_n = S0 Diag(e^G_n) + U^T Kt, and the gradients are
//   Z = Bm^T dO, E = dO^T Qa - Z^T W                    (before the scan)
//   dS_start = dS_end (Diag(e^G_n) - Kt^T W) + E         (reverse scan)
//   dU = Z + Kt dS_n^T, dBm = lower(dO U^T), dQp = dBm Km, dQa = dO S0,
//   dKm = dBm^T Qp + dL^T B Kp, dKt = U dS_n, dW = -dU S0,
//   dA = dW X^T + dU Y^T, dX = A^T dW, dY = A^T dU,
//   dL = strict_lower(-A^T dA A^T), dKp = B dL Km,
// then per element the chain through the decay factors and a reverse
// cumulative sum over rows gives d(log a), and d(alpha) = d(log a) / alpha.
//
// Structure: the forward prefill (snapshots every 64 tokens) supplies every
// chunk's start state; then per (chunk, head) unit, all units in parallel:
// prep (factors), one batched fp32 MFMA GEMM per product (64 x 64 output tiles
// staged through LDS), the 64 x 64 unit-lower inverse (one column per lane);
// the reverse scan over chunks per (sequence, head) keeps dS^T in MFMA
// accumulator registers (one 16-column slice per wavefront); a final kernel
// assembles dq, dk, dv, dalpha and dbeta. Everything is fp32 (16x16x4 fp32
// MFMA); a padded row of a short chunk has q = k = v = dO = 0, beta = 0 and
// no decay, which leaves every product unchanged.
#include "kda_internal.h"

namespace kda {
namespace {

using namespace bwd;
constexpr int C = 64;  // chunk length

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* base, int64_t idx) {
  if constexpr (BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[idx]);
  else return static_cast<const float*>(base)[idx];
}

// chunk_base[n] = sum over earlier sequences of ceil(len / 64) (chunks);
// snap_base[n] = the same of floor(len / 64) (64-token state slots);
// item_base[n] = the same of the scan segments, max(1, ceil(chunks / seg)).
__device__ __forceinline__ int64_t seq_items(int64_t nch, int32_t seg) {
  const int64_t it = seg > 0 ? (nch + seg - 1) / seg : 1;
  return it > 0 ? it : 1;
}

__global__ __launch_bounds__(1024) void chunk_base_kernel(const int64_t* cu, int32_t N, int32_t seg,
                                                          int64_t* chunk_base, int64_t* snap_base,
                                                          int64_t* item_base) {
  __shared__ int64_t pc[1024], ps[1024], pi[1024];
  const int tid = threadIdx.x;
  const int64_t per = ((int64_t)N + 1023) / 1024;
  const int64_t n0 = tid * per, n1 = n0 + per < (int64_t)N ? n0 + per : (int64_t)N;
  int64_t sc = 0, ss = 0, si = 0;
  for (int64_t n = n0; n < n1; ++n) {
    const int64_t len = cu[n + 1] - cu[n];
    sc += (len + C - 1) / C;
    ss += len / C;
    si += seq_items((len + C - 1) / C, seg);
  }
  pc[tid] = sc;
  ps[tid] = ss;
  pi[tid] = si;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int64_t vc = tid >= off ? pc[tid - off] : 0, vs = tid >= off ? ps[tid - off] : 0,
                  vi = tid >= off ? pi[tid - off] : 0;
    __syncthreads();
    pc[tid] += vc;
    ps[tid] += vs;
    pi[tid] += vi;
    __syncthreads();
  }
  int64_t bc = pc[tid] - sc, bs = ps[tid] - ss, bi = pi[tid] - si;
  for (int64_t n = n0; n < n1; ++n) {
    chunk_base[n] = bc;
    snap_base[n] = bs;
    item_base[n] = bi;
    const int64_t len = cu[n + 1] - cu[n];
    bc += (len + C - 1) / C;
    bs += len / C;
    bi += seq_items((len + C - 1) / C, seg);
  }
  if (tid == 1023) {
    chunk_base[N] = pc[1023];
    snap_base[N] = ps[1023];
    item_base[N] = pi[1023];
  }
}

struct ChunkPos {
  int32_t n, len;
  int64_t c, t0;
};
// The sequence holding chunk ch: the last n with chunk_base[n] <= ch (empty
// sequences share their successor's base and are skipped that way).
__device__ __forceinline__ ChunkPos chunk_pos(const BackwardArgs& a, int64_t ch) {
  int lo = 0, hi = a.num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.chunk_base[mid] <= ch) lo = mid; else hi = mid - 1;
  }
  ChunkPos p;
  p.n = lo;
  p.c = ch - a.chunk_base[lo];
  p.t0 = a.cu_dev[lo] + C * p.c;
  const int64_t rem = a.cu_dev[lo + 1] - p.t0;
  p.len = (int32_t)(rem < C ? rem : C);
  return p;
}

__device__ __forceinline__ int ref_row(int len) { return (len < 32 ? len : 32) - 1; }

// ---- prep: decay factors, scaled operands, the chunk's start state ---------
template <int D, bool BF16, bool PER_KEY>
__global__ __launch_bounds__(256) void prep_kernel(BackwardArgs a) {
  constexpr int LDG = D + 1;
  __shared__ float sG[C * LDG];
  __shared__ float sB[C];
  const int64_t units = a.n_chunks * a.H;
  const int64_t b = blockIdx.x;
  const int h = (int)(b % a.H);
  const ChunkPos p = chunk_pos(a, b / a.H);
  const int tid = threadIdx.x;
  if (tid < D) {                        // Gamma per channel: running sum of ln alpha
    float g = 0.f;
    for (int r = 0; r < C; ++r) {
      if (r < p.len) {
        const int64_t t = p.t0 + r;
        g += __logf(PER_KEY ? a.alpha[(t * a.H + h) * D + tid] : a.alpha[t * a.H + h]);
      }
      sG[r * LDG + tid] = g;
    }
  }
  if (tid < C) sB[tid] = tid < p.len ? a.beta[(p.t0 + tid) * a.H + h] : 0.f;
  __syncthreads();
  const int cref = ref_row(p.len);
  float* ws = a.ws;
  // four consecutive channels per thread: 8-byte bf16 (16-byte fp32) loads
  // and 16-byte stores
  for (int i4 = tid; i4 < C * D / 4; i4 += 256) {
    const int idx = 4 * i4, r = idx / D, j = idx % D;
    f32x4 qv = {0.f, 0.f, 0.f, 0.f}, kv = qv, vv = qv, dov = qv;
    if (r < p.len) {
      const int64_t e = ((p.t0 + r) * a.H + h) * D + j;
      qv = load4<BF16>(a.q, e);
      kv = load4<BF16>(a.k, e);
      vv = load4<BF16>(a.v, e);
      dov = *reinterpret_cast<const f32x4*>(a.d_o + e);
    }
    const float be = sB[r];
    f32x4 kp, km, qp, xa, qa, kt, yb, xp, gg;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float G = sG[r * LDG + j + i], Gc = sG[cref * LDG + j + i], Gn = sG[(C - 1) * LDG + j + i];
      const float eRel = __expf(G - Gc), eInv = __expf(Gc - G), eAbs = __expf(G), eTail = __expf(Gn - G);
      kp[i] = kv[i] * eRel;
      km[i] = kv[i] * eInv;
      qp[i] = qv[i] * eRel;
      xa[i] = be * (kv[i] * eAbs);
      qa[i] = qv[i] * eAbs;
      kt[i] = kv[i] * eTail;
      yb[i] = be * vv[i];
      xp[i] = be * (kv[i] * eRel);
      gg[i] = G;
    }
    const int64_t o = b * C * D + idx;
    auto st = [&](int arr, f32x4 x) { *reinterpret_cast<f32x4*>(ws + nd_off(arr, units, D) + o) = x; };
    st(KP, kp);
    st(KM, km);
    st(QP, qp);
    st(XA, xa);
    st(QA, qa);
    st(KT, kt);
    st(YB, yb);
    st(DOF, dov);
    st(XP, xp);
    st(GG, gg);
  }
  if (tid < D) ws[egn_off(units, D) + b * D + tid] = __expf(sG[(C - 1) * LDG + tid]);
  if (tid < C) ws[beta_off(units, D) + b * C + tid] = sB[tid];
  // start state of the chunk: the initial state (or 0) for a sequence's first
  // chunk, else the forward state after its first 64 c tokens
  const float* src = nullptr;
  if (p.c == 0) {
    if (a.init) src = a.init + ((int64_t)p.n * a.H + h) * D * D;
  } else {
    if (a.s0_in_place) return;          // (uniform) the forward wrote it in place
    src = a.states + ((a.snap_base[p.n] + p.c - 1) * a.H + h) * D * D;
  }
  float* dst = ws + dd_off(S0M, units, D) + b * D * D;
  for (int e = tid * 4; e < D * D; e += 1024)
    *reinterpret_cast<f32x4*>(dst + e) = src ? *reinterpret_cast<const f32x4*>(src + e) : f32x4{0.f, 0.f, 0.f, 0.f};
}

// ---- batched GEMM: C_b = alpha op(A_b) op(B_b) (+ C_b), fp32 MFMA ----------
struct GemmArgs {
  const float *A, *B;
  float* C;
  const float* rs;           // per-row scale of the product (or null)
  int64_t sA, sB, sC, srs;   // per-unit strides
  int32_t lda, ldb, ldc, M, N, K;
  float alpha;
  int32_t accumulate;        // add into C
  int32_t mask;              // 0: none, 1: keep row > col, 2: keep row >= col
  // optional second product of the same transposition, added before the
  // epilogue: C = alpha (op(A) op(B) + ratio2 op(A2) op(B2)) (ratio2 = +-1)
  const float *A2, *B2;
  int64_t sA2, sB2;
  int32_t lda2, ldb2, K2;
  float ratio2;
};

// One workgroup = one 64 x 64 output tile of one unit; four wavefronts of 16
// rows. C's ldc, its column offsets and its base are multiples of 4 floats. K advances in blocks of 32 staged in LDS: A as [m][k] (row stride 36)
// and B as [k][n] (row stride 80), strides that put the 64 lanes of each
// operand read on distinct banks.
template <bool TA, bool TB>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  constexpr int KB = 32, LDA = 36, LDB = 80;
  __shared__ float As[64 * LDA];
  __shared__ float Bs[KB * LDB];
  const int tn = g.N / 64, tiles = (g.M / 64) * tn;
  const int64_t b = blockIdx.x / tiles;
  const int tile = (int)(blockIdx.x % tiles);
  const int m0 = (tile / tn) * 64, n0 = (tile % tn) * 64;
  float* Cp = g.C + b * g.sC;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, gq = lane >> 4;
  f32x4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int term = 0; term < (g.A2 ? 2 : 1); ++term) {
    const float* A = term == 0 ? g.A + b * g.sA : g.A2 + b * g.sA2;
    const float* B = term == 0 ? g.B + b * g.sB : g.B2 + b * g.sB2;
    const int lda = term == 0 ? g.lda : g.lda2, ldb = term == 0 ? g.ldb : g.ldb2;
    const int K = term == 0 ? g.K : g.K2;
    const float sc = term == 0 ? 1.f : g.ratio2;      // applied to A while staging (exact for +-1)
    for (int k0 = 0; k0 < K; k0 += KB) {
#pragma unroll
      for (int e = tid; e < 512; e += 256) {
        if constexpr (!TA) {
          const int r = e >> 3, c = (e & 7) * 4;
          *reinterpret_cast<f32x4*>(As + r * LDA + c) =
              sc * *reinterpret_cast<const f32x4*>(A + (int64_t)(m0 + r) * lda + k0 + c);
        } else {
          const int kk = e >> 4, c = (e & 15) * 4;
          const f32x4 v = *reinterpret_cast<const f32x4*>(A + (int64_t)(k0 + kk) * lda + m0 + c);
#pragma unroll
          for (int i = 0; i < 4; ++i) As[(c + i) * LDA + kk] = sc * v[i];
        }
        if constexpr (!TB) {
          const int kk = e >> 4, c = (e & 15) * 4;
          *reinterpret_cast<f32x4*>(Bs + kk * LDB + c) =
              *reinterpret_cast<const f32x4*>(B + (int64_t)(k0 + kk) * ldb + n0 + c);
        } else {
          const int n = e >> 3, c = (e & 7) * 4;
          const f32x4 v = *reinterpret_cast<const f32x4*>(B + (int64_t)(n0 + n) * ldb + k0 + c);
#pragma unroll
          for (int i = 0; i < 4; ++i) Bs[(c + i) * LDB + n] = v[i];
        }
      }
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < KB / 4; ++ks) {
        const float av = As[(16 * w + l16) * LDA + 4 * ks + gq];
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = mfma4(Bs[(4 * ks + gq) * LDB + 16 * t + l16], av, acc[t]);
      }
      __syncthreads();
    }
  }
  // the tiles were formed transposed (B as the MFMA's first operand), so a
  // lane holds 4 consecutive columns of one row: one 16-byte store per tile
  const int row = m0 + 16 * w + l16;
  const float rsc = g.rs ? g.rs[b * g.srs + row] : 1.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int col0 = n0 + 16 * t + 4 * gq;
    f32x4 x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = g.alpha * acc[t][i];
      if ((g.mask == 1 && row <= col0 + i) || (g.mask == 2 && row < col0 + i)) x[i] = 0.f;
      if (g.rs) x[i] *= rsc;
    }
    f32x4* cp = reinterpret_cast<f32x4*>(Cp + (int64_t)row * g.ldc + col0);
    *cp = g.accumulate ? *cp + x : x;
  }
}

// ---- (I + L)^-1 with L = strict_lower(Diag(beta) P): one column per lane --
__global__ __launch_bounds__(64) void inverse_kernel(BackwardArgs a, int32_t d) {
  __shared__ float Ls[C * (C + 1)];
  const int64_t units = a.n_chunks * a.H, b = blockIdx.x;
  const float* P = a.ws + nn_off(PM, units, d) + b * C * C;
  const float* beta = a.ws + beta_off(units, d) + b * C;
  float* Ao = a.ws + nn_off(AM, units, d) + b * C * C;
  const int j = threadIdx.x;
  for (int r = 0; r < C; ++r) Ls[r * (C + 1) + j] = j < r ? beta[r] * P[r * C + j] : 0.f;
  __syncthreads();
  float x[C];
#pragma unroll
  for (int i = 0; i < C; ++i) {        // forward substitution down column j
    float s = i == j ? 1.f : 0.f;
#pragma unroll
    for (int m = 0; m < i; ++m) s -= Ls[i * (C + 1) + m] * x[m];
    x[i] = s;
  }
#pragma unroll
  for (int i = 0; i < C; ++i) Ao[i * C + j] = x[i];
}

// ---- reverse scan over chunks: dS_start = dS_end (Diag(e^G_n) - Kt^T W) + E ----
// Works on R = dS^T (d_k x d_v): R_start = Diag(e^G_n) R_end - W^T (Kt R_end) + E^T,
// and every column of R evolves on its own. Wavefront w owns columns
// 16w..16w+15 as D/16 accumulator tiles: lane (g, l) holds R(16t + 4g + i, 16w + l),
// i.e. dS(16w + l, 16t + 4g + i). Both products contract over the tile rows,
// which enter as the permuted-K operand. One workgroup runs one segment of
// one (sequence, head): OUT mode from the segment's true end gradient, storing
// dS at every chunk end (and d_initial at a sequence's first segment); MAP
// mode, for a sequence cut into segments, one of two chains per workgroup:
// from the identity without E (the segment's M) or from zero with E (its N),
// so that R_start = M R_end + N.
__device__ __forceinline__ int item_seq(const BackwardArgs& a, int64_t item) {
  int lo = 0, hi = a.num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.item_base[mid] <= item) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Three-term bf16 products: Kt and W^T are staged in LDS as bf16 hi + lo
// (hi = bf16(x), lo = bf16(x - hi)), and R and V1 enter as hi + lo pairs of
// their accumulator tiles (the permuted-K operand: lane group g supplies rows
// 4g..4g+3 of two consecutive 16-row tiles), so each 16x16x32 product is
// hi*hi + hi*lo + lo*hi (about 16 significant bits) accumulated in fp32.
__device__ __forceinline__ void split_pair_bf16(f32x4 t0, f32x4 t1, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = (__bf16)t0[i];
    lo[i] = (__bf16)(t0[i] - (float)hi[i]);
    hi[4 + i] = (__bf16)t1[i];
    lo[4 + i] = (__bf16)(t1[i] - (float)hi[4 + i]);
  }
}
// elements k0 + 4g .. +3 and k0 + 16 + 4g .. +3 of one bf16 row
__device__ __forceinline__ bf16x8 ld_perm_bf16(const __bf16* row, int k0, int gq) {
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  const bf16x4_t x0 = *reinterpret_cast<const bf16x4_t*>(row + k0 + 4 * gq);
  const bf16x4_t x1 = *reinterpret_cast<const bf16x4_t*>(row + k0 + 16 + 4 * gq);
  return bf16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
}
__device__ __forceinline__ f32x4 mfma3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, c, 0, 0, 0);
}

template <int D, bool MAP>
__global__ __launch_bounds__(D * 4) void scan_kernel(BackwardArgs a) {
  constexpr int LDK = D + 8;                       // Kt hi/lo: [chunk row][d_k]
  constexpr int LDW = C + 8;                       // W^T hi/lo: [d_k][chunk row]
  constexpr int NT = D / 16;                       // accumulator tiles per chain
  constexpr int PF = C * D / 4 / (D * 4);          // float4 of Kt (and of W) per thread per chunk
  __shared__ __bf16 KtH[C * LDK], KtL[C * LDK];
  __shared__ __bf16 WtH[D * LDW], WtL[D * LDW];
  const int chain = MAP ? (int)(blockIdx.x & 1) : 0;      // MAP: 0 = M, 1 = N
  const int64_t unit = MAP ? blockIdx.x >> 1 : blockIdx.x;
  const int64_t item = unit / a.H;
  const int h = (int)(unit % a.H);
  const int n = item_seq(a, item);
  const int64_t seg = item - a.item_base[n];
  const int64_t n_seg = a.item_base[n + 1] - a.item_base[n];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, gq = lane >> 4;
  const int64_t units = a.n_chunks * a.H, DD = (int64_t)D * D;
  const int64_t rowoff = (int64_t)(16 * w + l16) * D;
  const int64_t cb = a.chunk_base[n], nch = a.chunk_base[n + 1] - cb;
  const int64_t c0 = a.seg_chunks > 0 ? seg * a.seg_chunks : 0;
  const int64_t c1 = a.seg_chunks > 0 && c0 + a.seg_chunks < nch ? c0 + a.seg_chunks : nch;

  f32x4 R[NT];
  if constexpr (MAP) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) R[t][i] = (chain == 0 && 16 * t + 4 * gq + i == 16 * w + l16) ? 1.f : 0.f;
  } else {
    // a split sequence's end gradients all come from seg_end (the last
    // segment's is d_final, copied there by segment_end_kernel): this launch
    // writes d_initial, which may be the d_final buffer
    const float* src = nullptr;
    if (n_seg > 1) src = a.seg_end + (item * a.H + h) * DD + rowoff;
    else if (a.d_final) src = a.d_final + ((int64_t)n * a.H + h) * DD + rowoff;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      R[t] = src ? *reinterpret_cast<const f32x4*>(src + 16 * t + 4 * gq) : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // the next chunk's Kt and W, fetched into registers while this one computes
  f32x4 pk[PF], pw[PF];
  auto fetch = [&](int64_t c) {
    const int64_t b = (cb + c) * a.H + h;
    const float* kt = a.ws + nd_off(KT, units, D) + b * C * D;
    const float* wm = a.ws + nd_off(WM, units, D) + b * C * D;
#pragma unroll
    for (int q = 0; q < PF; ++q) {
      const int e = tid + q * D * 4;
      pk[q] = *reinterpret_cast<const f32x4*>(kt + (int64_t)(e / (D / 4)) * D + (e % (D / 4)) * 4);
      pw[q] = *reinterpret_cast<const f32x4*>(wm + (int64_t)(e / (D / 4)) * D + (e % (D / 4)) * 4);
    }
  };
  if (c1 > c0) fetch(c1 - 1);
  for (int64_t c = c1 - 1; c >= c0; --c) {
    const int64_t b = (cb + c) * a.H + h;
    if constexpr (!MAP) {
      float* dsn = a.ws + dd_off(DSN, units, D) + b * DD + rowoff;
#pragma unroll
      for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4*>(dsn + 16 * t + 4 * gq) = R[t];
    }
#pragma unroll
    for (int q = 0; q < PF; ++q) {
      const int e = tid + q * D * 4;
      const int r = e / (D / 4), c4 = (e % (D / 4)) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const __bf16 kh = (__bf16)pk[q][i], wh = (__bf16)pw[q][i];
        KtH[r * LDK + c4 + i] = kh;
        KtL[r * LDK + c4 + i] = (__bf16)(pk[q][i] - (float)kh);
        WtH[(c4 + i) * LDW + r] = wh;
        WtL[(c4 + i) * LDW + r] = (__bf16)(pw[q][i] - (float)wh);
      }
    }
    // R as hi + lo permuted-K operands (K = d_k in steps of 32)
    bf16x8 rh[D / 32], rl[D / 32];
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) split_pair_bf16(R[2 * ks], R[2 * ks + 1], rh[ks], rl[ks]);
    __syncthreads();
    if (c > c0) fetch(c - 1);
    const float* E = a.ws + dd_off(EM, units, D) + b * DD + rowoff;
    const float* eg = a.ws + egn_off(units, D) + b * D;
    f32x4 V1[4];                                    // Kt R: chunk rows 16s.., columns 16w..
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      V1[s] = f32x4{0.f, 0.f, 0.f, 0.f};
      const __bf16* kh = KtH + (16 * s + l16) * LDK;
      const __bf16* kl = KtL + (16 * s + l16) * LDK;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        V1[s] = mfma3(ld_perm_bf16(kh, 32 * ks, gq), ld_perm_bf16(kl, 32 * ks, gq), rh[ks], rl[ks], V1[s]);
    }
    bf16x8 vh[2], vl[2];                            // V1 as operand (K = chunk rows, 2 steps)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) split_pair_bf16(V1[2 * ks], V1[2 * ks + 1], vh[ks], vl[ks]);
    const bool with_e = !MAP || chain == 1;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      const __bf16* wh = WtH + (16 * t + l16) * LDW;
      const __bf16* wl = WtL + (16 * t + l16) * LDW;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        x = mfma3(ld_perm_bf16(wh, 32 * ks, gq), ld_perm_bf16(wl, 32 * ks, gq), vh[ks], vl[ks], x);
      const f32x4 gv = *reinterpret_cast<const f32x4*>(eg + 16 * t + 4 * gq);
      const f32x4 ev = with_e ? *reinterpret_cast<const f32x4*>(E + 16 * t + 4 * gq) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) R[t][i] = gv[i] * R[t][i] - x[i] + ev[i];
    }
    __syncthreads();
  }
  if constexpr (MAP) {
    float* m = a.seg_maps + (item * a.H + h) * 2 * DD + chain * DD + rowoff;
#pragma unroll
    for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4*>(m + 16 * t + 4 * gq) = R[t];
  } else if (seg == 0 && a.d_init) {
    float* di = a.d_init + ((int64_t)n * a.H + h) * DD + rowoff;
#pragma unroll
    for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4*>(di + 16 * t + 4 * gq) = R[t];
  }
}

// End gradient of every segment but the last, from the segment maps, in
// reverse: R_end(s) = M_{s+1} R_end(s+1) + N_{s+1}, R_end(last) = d_final^T.
// Same layout as the scan; M is read straight from memory as the A operand.
template <int D>
__global__ __launch_bounds__(D * 4) void segment_end_kernel(BackwardArgs a) {
  constexpr int NT = D / 16, LD = D + 4;
  __shared__ float Ms[D * LD];
  const int n = (int)(blockIdx.x / a.H), h = (int)(blockIdx.x % a.H);
  const int64_t ib = a.item_base[n], ns = a.item_base[n + 1] - ib;
  if (ns < 2) return;                       // uniform over the workgroup
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, gq = lane >> 4;
  const int64_t DD = (int64_t)D * D, rowoff = (int64_t)(16 * w + l16) * D;
  f32x4 R[NT];
  const float* df = a.d_final ? a.d_final + ((int64_t)n * a.H + h) * DD + rowoff : nullptr;
#pragma unroll
  for (int t = 0; t < NT; ++t) R[t] = df ? *reinterpret_cast<const f32x4*>(df + 16 * t + 4 * gq) : f32x4{0.f, 0.f, 0.f, 0.f};
  {
    // the last segment's own slot (otherwise unused) takes d_final, so that the
    // output scan never reads d_final while it writes d_initial
    float* e = a.seg_end + ((ib + ns - 1) * a.H + h) * DD + rowoff;
#pragma unroll
    for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4*>(e + 16 * t + 4 * gq) = R[t];
  }
  for (int64_t s = ns - 1; s >= 1; --s) {
    // maps are stored as the scan stores dS: element (r, c) of M at [c * D + r]
    const float* M = a.seg_maps + ((ib + s) * a.H + h) * 2 * DD;
    const float* N = M + DD + rowoff;
    for (int e = tid; e < D * D / 4; e += D * 4) {
      const int r = e / (D / 4), c4 = (e % (D / 4)) * 4;
      *reinterpret_cast<f32x4*>(Ms + r * LD + c4) = *reinterpret_cast<const f32x4*>(M + (int64_t)r * D + c4);
    }
    __syncthreads();
    f32x4 X[NT];
#pragma unroll
    for (int t2 = 0; t2 < NT; ++t2) {
      X[t2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) X[t2] = mfma4(Ms[(16 * t + 4 * gq + i) * LD + 16 * t2 + l16], R[t][i], X[t2]);
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const f32x4 nv = *reinterpret_cast<const f32x4*>(N + 16 * t + 4 * gq);
#pragma unroll
      for (int i = 0; i < 4; ++i) R[t][i] = X[t][i] + nv[i];
    }
    float* e = a.seg_end + ((ib + s - 1) * a.H + h) * DD + rowoff;
#pragma unroll
    for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4*>(e + 16 * t + 4 * gq) = R[t];
  }
}

// ---- assembly: dq, dk, dv, dbeta, and dalpha through the decay factors ----
// Every element (row r, channel j) in parallel: dq, dk, dv and the row's
// dGamma term, with the decay factors formed again from q, k and Gamma (the
// same expressions as the prep, so the same values); dGamma goes to LDS. The
// gradient of Gamma_n (which every row's log-decay contains) and dbeta are
// reductions over rows or channels; a last pass per channel sums dGamma over
// rows in reverse, which is the gradient of log alpha.
template <int D, bool BF16, bool PER_KEY>
__global__ __launch_bounds__(256) void assemble_kernel(BackwardArgs a) {
  constexpr int CQ = D / 4, RG = 256 / CQ;     // a thread owns 4 channels; RG threads share them
  constexpr int LDG = D + 4;
  __shared__ float sdG[C * LDG];
  __shared__ float sPart[RG * D];
  __shared__ float sGn[D];
  __shared__ float sBp[C * CQ];                 // per row, per channel quad: dY*V + dX*Ka
  const int64_t units = a.n_chunks * a.H;
  const int64_t b = blockIdx.x;
  const int h = (int)(b % a.H);
  const ChunkPos p = chunk_pos(a, b / a.H);
  const int tid = threadIdx.x;
  const float* ws = a.ws;
  auto nd = [&](int arr) { return ws + nd_off(arr, units, D) + b * C * D; };
  auto nn = [&](int arr) { return ws + nn_off(arr, units, D) + b * C * C; };
  auto ld4 = [](const float* p_) { return *reinterpret_cast<const f32x4*>(p_); };
  const float* beta = ws + beta_off(units, D) + b * C;
  const float *G = nd(GG), *dQp = nd(DQP), *dQa = nd(DQA), *dKp = nd(DKP), *dKm = nd(DKM), *dX = nd(DX),
              *dKt = nd(DKT), *dY = nd(DY);
  const int cref = ref_row(p.len);
  const int j4 = 4 * (tid % CQ), rg = tid / CQ;
  {                                     // elementwise part, four channels per thread
    const f32x4 Gc = ld4(G + cref * D + j4), Gn = ld4(G + (C - 1) * D + j4);
    f32x4 kt_part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int r = rg; r < C; r += RG) {
      const int e = r * D + j4;
      f32x4 qv = {0.f, 0.f, 0.f, 0.f}, kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      int64_t o = 0;
      if (r < p.len) {
        o = ((p.t0 + r) * a.H + h) * D + j4;
        qv = load4<BF16>(a.q, o);
        kv = load4<BF16>(a.k, o);
        vv = load4<BF16>(a.v, o);
      }
      const f32x4 g = ld4(G + e), dqp = ld4(dQp + e), dqa = ld4(dQa + e), dkp = ld4(dKp + e), dkm = ld4(dKm + e),
                  dx = ld4(dX + e), dkt = ld4(dKt + e), dy = ld4(dY + e);
      const float br = beta[r];
      f32x4 dG, dq, dk;
      float bpart = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float eRel = __expf(g[i] - Gc[i]), eInv = __expf(Gc[i] - g[i]), eAbs = __expf(g[i]),
                    eTail = __expf(Gn[i] - g[i]);
        const float dKa = br * dx[i];
        const float kt = kv[i] * eTail;
        dG[i] = dqp[i] * (qv[i] * eRel) + dqa[i] * (qv[i] * eAbs) + dkp[i] * (kv[i] * eRel) -
                dkm[i] * (kv[i] * eInv) + dKa * (kv[i] * eAbs) - dkt[i] * kt;
        kt_part[i] += dkt[i] * kt;
        dq[i] = dqp[i] * eRel + dqa[i] * eAbs;
        dk[i] = dkp[i] * eRel + dkm[i] * eInv + dKa * eAbs + dkt[i] * eTail;
        bpart += dy[i] * vv[i] + dx[i] * (kv[i] * eAbs);
      }
      *reinterpret_cast<f32x4*>(sdG + r * LDG + j4) = dG;
      sBp[r * CQ + j4 / 4] = bpart;
      if (r < p.len) {
        *reinterpret_cast<f32x4*>(a.dq + o) = dq;
        *reinterpret_cast<f32x4*>(a.dk + o) = dk;
        *reinterpret_cast<f32x4*>(a.dv + o) = br * dy;
      }
    }
    // gradient of Gamma_n: sum over rows of dKt * Kt, and colsum(dS_n * S0) e^Gamma_n
    const float* dSn = ws + dd_off(DSN, units, D) + b * D * D;
    const float* S0 = ws + dd_off(S0M, units, D) + b * D * D;
    f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int i = rg; i < D; i += RG) st += ld4(dSn + (int64_t)i * D + j4) * ld4(S0 + (int64_t)i * D + j4);
    *reinterpret_cast<f32x4*>(sPart + rg * D + j4) = kt_part + st * ld4(ws + egn_off(units, D) + b * D + j4);
  }
  __syncthreads();
  {                                     // dbeta: four lanes per row
    const int r = tid >> 2, part = tid & 3;
    const float *dL = nn(DLM), *P = nn(PM);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = part * 16; i < part * 16 + 16; i += 4) acc += ld4(dL + r * C + i) * ld4(P + r * C + i);
    float s = acc[0] + acc[1] + acc[2] + acc[3];
    for (int q = part * (CQ / 4); q < (part + 1) * (CQ / 4); ++q) s += sBp[r * CQ + q];
    s += __shfl_xor(s, 1, 4);
    s += __shfl_xor(s, 2, 4);
    if (part == 0 && r < p.len) a.dbeta[(p.t0 + r) * a.H + h] = s;
  }
  __syncthreads();
  if (tid < D) {
    float acc = 0.f;
#pragma unroll
    for (int q = 0; q < RG; ++q) acc += sPart[q * D + tid];
    sGn[tid] = acc;
  }
  __syncthreads();
  if (tid < D) {                        // reverse cumulative sum over rows
    float acc = sGn[tid];
    for (int r = C - 1; r >= 0; --r) {
      acc += sdG[r * LDG + tid];
      sdG[r * LDG + tid] = acc;
    }
  }
  __syncthreads();
  if constexpr (PER_KEY) {
    for (int idx = tid; idx < p.len * CQ; idx += 256) {
      const int r = idx / CQ, jj = 4 * (idx % CQ);
      const int64_t o = ((p.t0 + r) * a.H + h) * D + jj;
      *reinterpret_cast<f32x4*>(a.dalpha + o) = ld4(sdG + r * LDG + jj) / ld4(a.alpha + o);
    }
  } else {
    if (tid < p.len) {
      float s = 0.f;
      for (int jj = 0; jj < D; ++jj) s += sdG[tid * LDG + jj];
      const int64_t th = (p.t0 + tid) * a.H + h;
      a.dalpha[th] = s / a.alpha[th];
    }
  }
}

struct Term2 {
  const float *A = nullptr, *B = nullptr;
  int lda = 0;
  int64_t sA = 0;
  int ldb = 0;
  int64_t sB = 0;
  int K = 0;
  float ratio = 1.f;
};

hipError_t gemm(bool ta, bool tb, int64_t units, int d, int M, int N, int K, const float* A, int lda, int64_t sA,
                const float* B, int ldb, int64_t sB, float* Cm, int ldc, int64_t sC, float alpha, bool accumulate,
                int mask, const float* rs, const Term2& t2, hipStream_t s) {
  GemmArgs g{A, B, Cm, rs, sA, sB, sC, C, lda, ldb, ldc, M, N, K, alpha, accumulate ? 1 : 0, mask,
             t2.A, t2.B, t2.sA, t2.sB, t2.lda, t2.ldb, t2.K, t2.ratio};
  (void)d;
  const dim3 grid((unsigned)(units * (M / 64) * (N / 64)));
  if (!ta && !tb) hipLaunchKernelGGL((gemm_kernel<false, false>), grid, dim3(256), 0, s, g);
  else if (!ta && tb) hipLaunchKernelGGL((gemm_kernel<false, true>), grid, dim3(256), 0, s, g);
  else if (ta && !tb) hipLaunchKernelGGL((gemm_kernel<true, false>), grid, dim3(256), 0, s, g);
  else hipLaunchKernelGGL((gemm_kernel<true, true>), grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

template <int D, bool BF16, bool PK>
hipError_t backward_t(const BackwardArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(chunk_base_kernel, dim3(1), dim3(1024), 0, s, a.cu_dev, a.num_seqs, a.seg_chunks,
                     a.chunk_base, a.snap_base, a.item_base);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t U = a.n_chunks * a.H;
  if (U > 0) {
    float* w = a.ws;
    auto ND = [&](int arr) { return w + nd_off(arr, U, D); };
    auto NN = [&](int arr) { return w + nn_off(arr, U, D); };
    auto DDp = [&](int arr) { return w + dd_off(arr, U, D); };
    const int64_t sND = (int64_t)C * D, sNN = (int64_t)C * C, sDD = (int64_t)D * D;
    hipLaunchKernelGGL((prep_kernel<D, BF16, PK>), dim3((unsigned)U), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
#define G_(...) if ((e = gemm(__VA_ARGS__, Term2{}, s)) != hipSuccess) return e
#define G2_(...) if ((e = gemm(__VA_ARGS__, s)) != hipSuccess) return e
    // forward quantities
    G_(false, true, U, D, C, C, D, ND(KP), D, sND, ND(KM), D, sND, NN(PM), C, sNN, 1.f, false, 0, nullptr);
    hipLaunchKernelGGL(inverse_kernel, dim3((unsigned)U), dim3(64), 0, s, a, (int32_t)D);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    G_(false, false, U, D, C, D, C, NN(AM), C, sNN, ND(XA), D, sND, ND(WM), D, sND, 1.f, false, 0, nullptr);
    G_(false, false, U, D, C, D, C, NN(AM), C, sNN, ND(YB), D, sND, ND(UM), D, sND, 1.f, false, 0, nullptr);
    G_(false, true, U, D, C, D, D, ND(WM), D, sND, DDp(S0M), D, sDD, ND(UM), D, sND, -1.f, true, 0, nullptr);
    G_(false, true, U, D, C, C, D, ND(QP), D, sND, ND(KM), D, sND, NN(BM), C, sNN, 1.f, false, 2, nullptr);
    // inputs of the reverse scan
    G_(true, false, U, D, C, D, C, NN(BM), C, sNN, ND(DOF), D, sND, ND(ZU), D, sND, 1.f, false, 0, nullptr);
    // E = dO^T Qa - Z^T W in one launch
    G2_(true, false, U, D, D, D, C, ND(DOF), D, sND, ND(QA), D, sND, DDp(EM), D, sDD, 1.f, false, 0, nullptr,
       Term2{ND(ZU), ND(WM), D, sND, D, sND, C, -1.f});
  }
  const dim3 scan_grid((unsigned)(a.n_items * a.H));
  if (a.seg_chunks > 0) {
    hipLaunchKernelGGL((scan_kernel<D, true>), dim3((unsigned)(a.n_items * a.H * 2)), dim3(D * 4), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((segment_end_kernel<D>), dim3((unsigned)((int64_t)a.num_seqs * a.H)), dim3(D * 4), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((scan_kernel<D, false>), scan_grid, dim3(D * 4), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (U > 0) {
    float* w = a.ws;
    auto ND = [&](int arr) { return w + nd_off(arr, U, D); };
    auto NN = [&](int arr) { return w + nn_off(arr, U, D); };
    auto DDp = [&](int arr) { return w + dd_off(arr, U, D); };
    const int64_t sND = (int64_t)C * D, sNN = (int64_t)C * C, sDD = (int64_t)D * D;
    // local gradients
    G_(false, true, U, D, C, D, D, ND(KT), D, sND, DDp(DSN), D, sDD, ND(ZU), D, sND, 1.f, true, 0, nullptr);
    G_(false, true, U, D, C, C, D, ND(DOF), D, sND, ND(UM), D, sND, NN(DBM), C, sNN, 1.f, false, 2, nullptr);
    G_(false, false, U, D, C, D, C, NN(DBM), C, sNN, ND(KM), D, sND, ND(DQP), D, sND, 1.f, false, 0, nullptr);
    G_(false, false, U, D, C, D, D, ND(DOF), D, sND, DDp(S0M), D, sDD, ND(DQA), D, sND, 1.f, false, 0, nullptr);
    G_(false, false, U, D, C, D, D, ND(UM), D, sND, DDp(DSN), D, sDD, ND(DKT), D, sND, 1.f, false, 0, nullptr);
    G_(false, false, U, D, C, D, D, ND(ZU), D, sND, DDp(S0M), D, sDD, ND(DW), D, sND, -1.f, false, 0, nullptr);
    // dA = dW X^T + dU Y^T in one launch
    G2_(false, true, U, D, C, C, D, ND(DW), D, sND, ND(XA), D, sND, NN(DAM), C, sNN, 1.f, false, 0, nullptr,
       Term2{ND(ZU), ND(YB), D, sND, D, sND, D, 1.f});
    G_(true, false, U, D, C, D, C, NN(AM), C, sNN, ND(DW), D, sND, ND(DX), D, sND, 1.f, false, 0, nullptr);
    G_(true, false, U, D, C, D, C, NN(AM), C, sNN, ND(ZU), D, sND, ND(DY), D, sND, 1.f, false, 0, nullptr);
    G_(false, true, U, D, C, C, C, NN(DAM), C, sNN, NN(AM), C, sNN, NN(TM), C, sNN, 1.f, false, 0, nullptr);
    G_(true, false, U, D, C, C, C, NN(AM), C, sNN, NN(TM), C, sNN, NN(DLM), C, sNN, -1.f, false, 1, nullptr);
    G_(false, false, U, D, C, D, C, NN(DLM), C, sNN, ND(KM), D, sND, ND(DKP), D, sND, 1.f, false, 0,
       w + beta_off(U, D));
    // dKm = dBm^T Qp + dL^T (B Kp) in one launch
    G2_(true, false, U, D, C, D, C, NN(DBM), C, sNN, ND(QP), D, sND, ND(DKM), D, sND, 1.f, false, 0, nullptr,
       Term2{NN(DLM), ND(XP), C, sNN, D, sND, C, 1.f});
#undef G_
#undef G2_
    hipLaunchKernelGGL((assemble_kernel<D, BF16, PK>), dim3((unsigned)U), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& a, int d, bool bf16, bool per_key, hipStream_t s) {
  if (d == 64) {
    if (bf16) return per_key ? backward_t<64, true, true>(a, s) : backward_t<64, true, false>(a, s);
    return per_key ? backward_t<64, false, true>(a, s) : backward_t<64, false, false>(a, s);
  }
  if (bf16) return per_key ? backward_t<128, true, true>(a, s) : backward_t<128, true, false>(a, s);
  return per_key ? backward_t<128, false, true>(a, s) : backward_t<128, false, false>(a, s);
}

}  // namespace kda
