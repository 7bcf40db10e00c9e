// kda_layer.hip — the front and back end of a KDA layer around the recurrence.
//
// Page "kda-graft: Qwen2.5-0.5B с трансплантированным KDA" (ailist.pro),
// section "Идея и архитектура": a KDA layer adds a 4-tap convolution
// initialised as an identity tap, an alpha gate with bias +5, beta, an output
// gate and RMSNorm. The page gives no formulas; this file computes
//   front:  q, k, v = SiLU(causal depthwise 4-tap conv over each sequence's
//           tokens, carried state before its first token), q and k
//           L2-normalised over d; alpha = sigmoid(logit + bias);
//           beta = sigmoid(logit); and the carried state after each sequence
//           (its last 3 conv inputs, oldest first);
//   back:   out = o * rsqrt(mean(o^2) + eps) * w * sigmoid(g) per (token, head).
// Both are streaming kernels: every input is read once and every output
// written once, so they are bound by HBM bandwidth.
//
// Mapping: a lane owns 8 consecutive channels, so a row's D channels span D/8
// lanes; the row's sums of squares are reduced across those lanes with xor
// shuffles. Sigmoids use the hardware reciprocal and bf16 stores the gfx950
// packed round-to-nearest-even conversion.
#include "kda_internal.h"

namespace kda {
namespace {

// One row segment of 8 channels as loaded: 16 bytes of bf16 or 32 bytes of fp32.
template <bool BF16> struct Raw8;
template <> struct Raw8<true> { uint4 w; };
template <> struct Raw8<false> { f32x4 a, b; };

template <bool BF16>
__device__ __forceinline__ void load_raw(const void* base, int64_t idx, Raw8<BF16>& r) {
  if constexpr (BF16) {
    r.w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
  } else {
    r.a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx);
    r.b = *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx + 4);
  }
}

template <bool BF16>
__device__ __forceinline__ void zero_raw(Raw8<BF16>& r) {
  if constexpr (BF16) r.w = uint4{0u, 0u, 0u, 0u};
  else r.a = r.b = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <bool BF16>
__device__ __forceinline__ float raw_at(const Raw8<BF16>& r, int e) {
  if constexpr (BF16) {
    const uint32_t u = e < 2 ? r.w.x : e < 4 ? r.w.y : e < 6 ? r.w.z : r.w.w;
    return __uint_as_float((e & 1) ? (u & 0xFFFF0000u) : (u << 16));
  } else {
    return e < 4 ? r.a[e] : r.b[e - 4];
  }
}

template <bool BF16>
__device__ __forceinline__ void load8(const void* base, int64_t idx, float (&x)[8]) {
  Raw8<BF16> r;
  load_raw<BF16>(base, idx, r);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = raw_at<BF16>(r, e);
}

template <bool BF16>
__device__ __forceinline__ void store8(void* base, int64_t idx, const float (&x)[8]) {
  if constexpr (BF16) {
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + idx) =
        uint4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx + 4) = f32x4{x[4], x[5], x[6], x[7]};
  }
}

// sum over the CG lanes (a power of two, lane-aligned) that share a row
template <int CG>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int m = 1; m < CG; m <<= 1) x += __shfl_xor(x, m, CG);
  return x;
}

__device__ __forceinline__ int seq_of(const int64_t* cu, int32_t num_seqs, int64_t t) {
  int lo = 0, hi = num_seqs - 1;                 // last n with cu[n] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

constexpr int kGroupsPerBlock = 64;             // 8-channel groups per workgroup: one per lane
constexpr int64_t kFrontLongRows = 32768;       // token rows from which a workgroup takes 8 tokens

// Front end. The token rows are [T, H*D]; a lane owns one group of 8
// consecutive channels, so one wavefront load reads 64 x 8 channels of a row
// in one contiguous piece (1 KB in bf16). A workgroup covers one block of 64
// channel groups for TPT consecutive tokens: one wavefront each for the q, k
// and v convolutions, and for the per-key gate (a [T, H, d] tensor in and
// out, as heavy as a convolution) a fourth one for the gates; the scalar
// gates (two values per token and head) are formed by the v wavefront after
// its stores, so every resident wavefront of a scalar-gate launch streams rows.
// Each wavefront issues all its loads (its TPT rows, the 3 rows before them
// and its taps) before its first store, so no wait on a load also waits on its
// own stores, and forms the 4-tap convolution in registers. The CG lanes of one
// (token, head) are an aligned lane group (H*CG groups per row, CG | 64), which
// the L2 norm reduces with shuffles.
template <bool PER_KEY, int TPT>
struct FrontGates {
  float al[TPT][PER_KEY ? 8 : 1], bl[TPT];
  __device__ __forceinline__ void load(const LayerFrontArgs& a, int64_t tfirst, int64_t HD, int64_t ch0, int h) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int64_t t = tfirst + i < a.T ? tfirst + i : a.T - 1;
      if constexpr (PER_KEY) load8<false>(a.alpha_logit, t * HD + ch0, al[i]);
      else al[i][0] = a.alpha_logit[t * a.H + h];
      bl[i] = a.beta_logit[t * a.H + h];
    }
  }
  __device__ __forceinline__ void store(const LayerFrontArgs& a, int64_t tfirst, int64_t HD, int64_t ch0, int h,
                                        bool live, bool lead) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int64_t t = tfirst + i;
      if (t >= a.T) break;
      if constexpr (PER_KEY) {
#pragma unroll
        for (int e = 0; e < 8; ++e) al[i][e] = sigmoid_rcp(al[i][e] + a.alpha_bias);
        if (live) store8<false>(a.alpha, t * HD + ch0, al[i]);
      } else {
        if (lead) a.alpha[t * a.H + h] = sigmoid_rcp(al[i][0] + a.alpha_bias);
      }
      if (lead) a.beta[t * a.H + h] = sigmoid_rcp(bl[i]);
    }
  }
};

template <bool PER_KEY>
constexpr int front_waves() { return PER_KEY ? 4 : 3; }

template <int D, bool BF16, bool PER_KEY, int TPT>
__global__ __launch_bounds__(256) void layer_front_kernel(LayerFrontArgs a, int32_t n_cblocks) {
  constexpr int CG = D / 8;
  const int lane = threadIdx.x & 63;
  const int j = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // 0, 1, 2: q, k, v; 3: gates
  // the channel blocks of one token tile are neighbours in launch order, so
  // whole rows are read at about the same time
  const int cblock = (int)(blockIdx.x % (uint32_t)n_cblocks);
  const int64_t tfirst = (int64_t)(blockIdx.x / (uint32_t)n_cblocks) * TPT;
  const int G = a.H * CG;
  const int g_raw = cblock * kGroupsPerBlock + lane;
  const bool live = g_raw < G;                   // whole aligned CG groups are live or not (CG | G, CG | 64)
  const int g = live ? g_raw : 0;                // dead lanes compute on group 0 and store nothing
  const int h = g / CG;
  const int64_t HD = (int64_t)a.H * D;
  const int64_t ch0 = (int64_t)g * 8;            // = h*D + 8*(g % CG)
  const bool lead = live && (g % CG) == 0;       // one lane per (token, head)

  FrontGates<PER_KEY, TPT> gates;
  if (PER_KEY && j == 3) {                       // gates
    gates.load(a, tfirst, HD, ch0, h);
    gates.store(a, tfirst, HD, ch0, h, live, lead);
    return;
  }

  const void* x = j == 0 ? a.xq : j == 1 ? a.xk : a.xv;
  void* y_out = j == 0 ? a.q : j == 1 ? a.k : a.v;
  Raw8<BF16> win[TPT + 3];                       // rows tfirst-3 .. tfirst+TPT-1
  if (tfirst >= 3 && tfirst + TPT <= a.T) {
#pragma unroll
    for (int r = 0; r < TPT + 3; ++r) load_raw<BF16>(x, (tfirst - 3 + r) * HD + ch0, win[r]);
  } else {
#pragma unroll
    for (int r = 0; r < TPT + 3; ++r) {
      const int64_t p = tfirst - 3 + r;
      if (p >= 0 && p < a.T) load_raw<BF16>(x, p * HD + ch0, win[r]);
      else zero_raw<BF16>(win[r]);
    }
  }
  if (!PER_KEY && j == 2) gates.load(a, tfirst, HD, ch0, h);   // before any store of this wavefront
  // Taps of the lane's 8 channels, oldest first. The wavefront's 8 KB (16 B
  // per channel) are read in whole 1 KB pieces and passed through LDS, where
  // lane l's 8 pieces sit in 8 consecutive 16-byte slots permuted by l mod 8,
  // so the 8 lanes of one read phase hit distinct banks. Only this wavefront
  // touches its slots: no workgroup barrier.
  f32x4 w[8];
  {
    __shared__ f32x4 tap_lds[3][kGroupsPerBlock * 8];
    const float* tb = a.conv_w + ((int64_t)j * HD + (int64_t)cblock * (kGroupsPerBlock * 8)) * 4;
    f32x4 pc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int u = e * 64 + lane;               // channel cblock*512 + u
      if (cblock * kGroupsPerBlock + u / 8 < G) pc[e] = *reinterpret_cast<const f32x4*>(tb + u * 4);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int u = e * 64 + lane, l = u / 8;
      if (cblock * kGroupsPerBlock + l < G) tap_lds[j][l * 8 + ((u % 8) ^ (l % 8))] = pc[e];
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = tap_lds[j][lane * 8 + (e ^ (lane % 8))];
  }

  // sequence of each token (wave-uniform, so scalar): last n with cu[n] <= t
  int seq[TPT];
  int64_t start[TPT];
  {
    int sq = seq_of(a.cu, a.num_seqs, tfirst);
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      while (sq + 1 < a.num_seqs && a.cu[sq + 1] <= tfirst + i) ++sq;
      seq[i] = sq;
      start[i] = a.cu[sq];
    }
  }

  float xr[TPT + 3][8];                          // unpacked once, used by up to 4 taps
#pragma unroll
  for (int r = 0; r < TPT + 3; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) xr[r][e] = raw_at<BF16>(win[r], e);

  // every window inside its token's sequence (start is nondecreasing in i):
  // the convolution needs neither the carried state nor zero padding
  const bool inside = start[TPT - 1] <= tfirst - 3;
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int64_t t = tfirst + i;
    float y[8];
    if (inside) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y[e] = w[e][0] * xr[i][e];
#pragma unroll
        for (int tap = 1; tap < 4; ++tap) y[e] += w[e][tap] * xr[i + tap][e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = 0.f;
#pragma unroll
      for (int tap = 0; tap < 4; ++tap) {
        const int64_t p = t - 3 + tap;
        if (p >= start[i]) {                     // wave-uniform: every lane has the same tokens
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] += w[e][tap] * xr[i + tap][e];
        } else if (a.conv_state_in != nullptr) {
          // carried input p - start + 3 of this sequence's state (oldest first)
          float xs[8];
          load8<BF16>(a.conv_state_in, (((int64_t)seq[i] * 3 + j) * 3 + (p - start[i] + 3)) * HD + ch0, xs);
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] += w[e][tap] * xs[e];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = y[e] * sigmoid_rcp(y[e]);            // SiLU
    if (j < 2) {                                                        // q, k: unit rows
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += y[e] * y[e];
      ss = row_sum<CG>(ss);
      const float r = __builtin_amdgcn_rsqf(ss + 1e-6f);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] *= r;
    }
    if (live && t < a.T) store8<BF16>(y_out, t * HD + ch0, y);
  }
  if (!PER_KEY && j == 2) gates.store(a, tfirst, HD, ch0, h, live, lead);
}

// Carried convolution state after each sequence: its last 3 inputs, oldest
// first, shifted in from the incoming state when the sequence is shorter.
// One thread per 8 channels of (sequence, q/k/v, tap, head).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void layer_conv_state_kernel(LayerFrontArgs a) {
  constexpr int CG = D / 8;
  const int64_t HD = (int64_t)a.H * D;
  const int64_t total = (int64_t)a.num_seqs * 3 * 3 * a.H * CG;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    int64_t rem = e;
    const int cg = rem % CG; rem /= CG;
    const int h = rem % a.H; rem /= a.H;
    const int tap = rem % 3; rem /= 3;
    const int j = rem % 3;
    const int n = (int)(rem / 3);
    const int64_t len = a.cu[n + 1] - a.cu[n];
    const int64_t ext = len + tap;               // index in [carried 3 inputs, sequence inputs]
    const int64_t ch0 = (int64_t)h * D + 8 * cg;
    float x[8];
    if (ext >= 3) {
      const void* src = j == 0 ? a.xq : j == 1 ? a.xk : a.xv;
      load8<BF16>(src, (a.cu[n] + ext - 3) * HD + ch0, x);
    } else if (a.conv_state_in != nullptr) {
      load8<BF16>(a.conv_state_in, (((int64_t)n * 3 + j) * 3 + ext) * HD + ch0, x);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = 0.f;
    }
    store8<BF16>(a.conv_state_out, (((int64_t)n * 3 + j) * 3 + tap) * HD + ch0, x);
  }
}

// The row's sum of squares: each lane's 8 values in order as fused
// multiply-adds, then the xor-pairwise sum over the row's lanes (the
// prefill's fused back end forms the same sum in the same order).
template <int D, bool OUT_BF16, bool G_BF16>
__global__ __launch_bounds__(256) void layer_back_kernel(LayerBackArgs a) {
  constexpr int CG = D / 8;
  constexpr int RPB = 256 / CG;                  // rows per workgroup
  const int cg = threadIdx.x % CG;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / CG;   // (token, head)
  const bool live = row < a.rows;
  const int64_t off = (live ? row : 0) * D + 8 * cg;
  float o[8], g[8], w[8];
  load8<false>(a.o, off, o);
  load8<G_BF16>(a.g_logit, off, g);
  load8<false>(a.norm_w, 8 * cg, w);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(o[e], o[e], ss);
  ss = row_sum<CG>(ss);
  const float r = __builtin_amdgcn_rsqf(ss / D + a.eps);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = o[e] * r * w[e] * sigmoid_rcp(g[e]);
  if (live) store8<OUT_BF16>(a.out, off, o);
}

template <int D, bool BF16, bool PK, int TPT>
hipError_t front_t(const LayerFrontArgs& a, hipStream_t s) {
  if (a.T > 0) {
    const int32_t n_cblocks = (a.H * (D / 8) + kGroupsPerBlock - 1) / kGroupsPerBlock;
    const int64_t tiles = (a.T + TPT - 1) / TPT;
    hipLaunchKernelGGL((layer_front_kernel<D, BF16, PK, TPT>), dim3((unsigned)(tiles * n_cblocks)),
                       dim3(64 * front_waves<PK>()), 0, s, a, n_cblocks);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.conv_state_out != nullptr && a.num_seqs > 0) {
    const int64_t total = (int64_t)a.num_seqs * 9 * a.H * (D / 8);
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL((layer_conv_state_kernel<D, BF16>), dim3((unsigned)(blocks < 65535 ? blocks : 65535)),
                       dim3(256), 0, s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

// 8 tokens per workgroup once there are enough rows to fill the chip (fewer
// halo re-reads), else 4
template <int D, bool BF16, bool PK>
hipError_t front_pick(const LayerFrontArgs& a, hipStream_t s) {
  if (a.T >= kFrontLongRows) return front_t<D, BF16, PK, 8>(a, s);
  return front_t<D, BF16, PK, 4>(a, s);
}

template <int D>
hipError_t back_t(const LayerBackArgs& a, bool out_bf16, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  constexpr int RPB = 256 / (D / 8);
  const dim3 grid((unsigned)((a.rows + RPB - 1) / RPB));
  if (a.g_bf16) {
    if (out_bf16) hipLaunchKernelGGL((layer_back_kernel<D, true, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((layer_back_kernel<D, false, true>), grid, dim3(256), 0, s, a);
  } else {
    if (out_bf16) hipLaunchKernelGGL((layer_back_kernel<D, true, false>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((layer_back_kernel<D, false, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_layer_front(const LayerFrontArgs& a, int d, bool bf16, bool per_key, hipStream_t s) {
  if (d == 64) {
    if (bf16) return per_key ? front_pick<64, true, true>(a, s) : front_pick<64, true, false>(a, s);
    return per_key ? front_pick<64, false, true>(a, s) : front_pick<64, false, false>(a, s);
  }
  if (bf16) return per_key ? front_pick<128, true, true>(a, s) : front_pick<128, true, false>(a, s);
  return per_key ? front_pick<128, false, true>(a, s) : front_pick<128, false, false>(a, s);
}

hipError_t launch_layer_back(const LayerBackArgs& a, int d, bool out_bf16, hipStream_t s) {
  return d == 64 ? back_t<64>(a, out_bf16, s) : back_t<128>(a, out_bf16, s);
}

}  // namespace kda
