// kda_prefill.hip — chunkwise-parallel prefill of the gated delta rule on gfx950.
//
// The update (page "Modele hybrydowe: co Gated DeltaNet zastępuje w cache KV",
// trefon.com, section "Gated DeltaNet: dodaj zanik") with the per-key-channel
// decay read as Diag(a_t) on the key axis:
//     S_t = S_{t-1} Diag(a_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t.
// The same page (closing paragraph of "Co stan rekurencyjny zmienia przy
// serwowaniu") states that inside a chunk the updates are dense matrix
// products and only chunk-to-chunk is sequential. For a chunk of n <= 64
// tokens with start state S0 and in-chunk cumulative log decay
// G_r = sum_{i<=r} log2 a_i (row r = token r, column = key channel):
//     L_ri = beta_r sum_j k_r[j] k_i[j] 2^(G_r[j]-G_i[j])   (i < r)
//     A    = (I + L)^-1,  T~ = A Diag(beta)                 (UT / WY form)
//     W    = T~ (K * 2^G),  U' = T~ V,  U = U' - W S0^T
//     O    = (Q * 2^G) S0^T + B U,  B_ri = sum_j q_r[j] k_i[j] 2^(G_r[j]-G_i[j]) (i <= r)
//     S_n  = S0 Diag(2^(G_n)) + U^T (K * 2^(G_n - G))
// so S_n = S0 M + N with M = Diag(2^G_n) - W^T (K*2^(G_n-G)) and
// N = U'^T (K*2^(G_n-G)): a chunk, and hence a run of chunks, acts on the
// state as an affine map.
//
// Kernel structure. One workgroup per (work item, head). The state
// (D = d_k = d_v rows) is cut into 16-row slices, one per wavefront at
// D = 128 (eight wavefronts, two per SIMD) and two per wavefront at D = 64
// (four wavefronts, one per SIMD); each wavefront keeps its slices
// transposed, S0^T, in MFMA accumulator layout (fp32) for the whole item.
// Per chunk:
//   P1  the decay cumsum G (fp32); beta; 2^G_n. bf16 q, k rows were staged
//       in LDS by the previous chunk and are read there directly by P2, P3;
//       fp32 inputs are copied to fp16 here.
//   P2  decayed operands in LDS: Q~ = Q*2^G [c][k], K^T*2^G and
//       (K*2^(G_n-G))^T [k][c] (fp16).
//   P3  Gram tile pairs on MFMA: L (fp32) and B (fp16). Scalar gate: exact
//       products K K^T, Q K^T of the inputs (bf16 MFMA on bf16 inputs, fp16
//       MFMA on the fp16 copy of fp32 ones) scaled by 2^(G_r-G_i) in fp32. Per-key
//       gate: three-term bf16 products (hi*hi + hi*lo + lo*hi) of operands
//       decayed relative to the first token of each 16-row block, so every
//       factor stays in fp32/bf16 range. Two wavefronts then invert the four
//       16x16 unit-lower diagonal blocks of I + L (right-looking
//       substitution, one column per lane).
//   P4  off-diagonal blocks of (I + L)^-1: one register-resident chain of
//       fp32 MFMA products per block column; V^T staged in LDS.
//   P5  T~ = (I + L)^-1 Diag(beta) split into fp16 hi + lo; W = T~ (K*2^G)
//       and U' = T~ V on MFMA from the same T~ tiles.
//   P6  per slice: U = U' - W S0^T, O^T = S0 Q~^T + U^T B^T (a lane then
//       holds four consecutive values of one token),
//       S0^T <- 2^(G_n) S0^T + (K*2^(G_n-G))^T U. U enters its products as
//       fp16 hi + lo; the state stays fp32. The next chunk's inputs are
//       fetched (q, k rows straight into LDS) while P6 runs.
// Three instantiations: OUT (the real chain: o, snapshots, final state), MAP
// (a segment's affine map: each wavefront advances its N rows, the chain from
// S0 = 0, and its M rows, the chain with v = 0 from identity rows, side by side;
// q, Q~, B and o are skipped) and WU (OUT for the segments of a split sequence).
// Long sequences with few heads are split into segments: pass 1 maps every
// segment and keeps each chunk's W and U' (the products of P5), a scan composes
// S_{s+1} = S_s M_s + N_s in fp32 from the initial state, and pass 3 (WU) runs
// every segment from its true start, loading W and U' instead of forming L,
// the inverse and P5 again; whole sequences of the same call run in OUT. For
// the scalar gate with bf16 inputs at d = 128, both passes are kernels of their
// own: in pass 1 (prefill_map_chain_kernel) four wavefronts carry the N rows
// while eight form the next chunk's state-free phases and carry the M rows; in
// pass 3 (prefill_wu_pipe_kernel) four wavefronts run the chain while the
// other four prepare the next chunk's operands. Pass 3 can also apply the KDA
// layer's back end (RMSNorm over d, norm weights, sigmoid output gate) to each
// chunk's output tile on chip and write the layer output instead of o: the
// chain wavefronts form each row's sum of squares in the order the separate
// back-end kernel does (same bits), the producers stage the gate logits and
// store the bf16 output rows through LDS, whole rows at a time.
// Accumulator layout of a 16x16 MFMA tile: lane l holds rows 4(l/16)+i,
// column l%16. When an accumulator tile feeds the next product as its
// K-operand, the K index is permuted (lane group g supplies rows 4g..4g+3 of
// each of two tiles) and the other operand is read with the same permutation,
// so no data moves between lanes.
#include <type_traits>

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int C = 64;  // chunk length

// Work item idx: from the table build_items_kernel writes, or, with one
// sequence, formed here exactly as that kernel would (segments of seg_chunks
// chunks, or the whole sequence).
__device__ __forceinline__ PrefillItem work_item(const PrefillArgs& a, int idx) {
  if (!a.one_seq) return a.items[idx];
  const int64_t st = (int64_t)a.seg_chunks * C;
  const bool split = st > 0 && a.one_len > st;
  PrefillItem it;
  it.n_segs = split ? (int32_t)((a.one_len + st - 1) / st) : 1;
  it.tok_in_seq = split ? (int64_t)idx * st : 0;
  it.tok_begin = a.one_tok0 + it.tok_in_seq;
  it.n_tokens = (int32_t)(split ? min(st, a.one_len - it.tok_in_seq) : a.one_len);
  it.snap_base = 0;
  it.seq = 0;
  it.seg = split ? idx : 0;
  return it;
}


__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

// Hardware base-2 exponential and logarithm (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// [k][c] fp16 arrays (K^T, K~^T, V^T) rotate each row by 8 * ((k / 16) % 8)
// columns. The transposed staging writes of 16 consecutive 8-channel groups
// then land on distinct LDS banks, and so do the operand reads of 16
// consecutive rows (one rotation per 16-row tile, rows 72 halves apart);
// aligned groups of 4 and 8 columns stay contiguous, which is all the MFMA
// operand reads need.
__device__ __forceinline__ int swz(int k, int c) { return (c + 8 * ((k >> 4) & 7)) & 63; }

// Row (l%16) of a row-major fp16 matrix, the 8 K-elements of lane group
// g = l/16 in the standard order: k0 + 8g .. k0 + 8g + 7.
__device__ __forceinline__ f16x8 ld_std(const _Float16* base, int ld, int row0, int k0, int lane) {
  return *reinterpret_cast<const f16x8*>(base + (row0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}
// Same row, permuted K order: k0 + 4g + {0..3}, then k0 + 16 + 4g + {0..3}.
__device__ __forceinline__ f16x8 ld_perm(const _Float16* base, int ld, int row0, int k0, int lane) {
  const _Float16* p = base + (row0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4);
  const f16x4 lo = *reinterpret_cast<const f16x4*>(p);
  const f16x4 hi = *reinterpret_cast<const f16x4*>(p + 16);
  return f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// The same two reads from a swizzled [k][c] array (row = k, K index = c).
__device__ __forceinline__ f16x8 ld_std_swz(const _Float16* base, int ld, int row0, int k0, int lane) {
  const int r = row0 + (lane & 15);
  return *reinterpret_cast<const f16x8*>(base + r * ld + swz(r, k0 + 8 * (lane >> 4)));
}
__device__ __forceinline__ f16x8 ld_perm_swz(const _Float16* base, int ld, int row0, int k0, int lane) {
  const int r = row0 + (lane & 15);
  const f16x4 lo = *reinterpret_cast<const f16x4*>(base + r * ld + swz(r, k0 + 4 * (lane >> 4)));
  const f16x4 hi = *reinterpret_cast<const f16x4*>(base + r * ld + swz(r, k0 + 16 + 4 * (lane >> 4)));
  return f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// Two accumulator tiles (rows k0..k0+15 and k0+16..k0+31) as a permuted-K operand.
__device__ __forceinline__ f16x8 pack_perm(f32x4 t0, f32x4 t1) {
  return f16x8{(_Float16)t0[0], (_Float16)t0[1], (_Float16)t0[2], (_Float16)t0[3],
               (_Float16)t1[0], (_Float16)t1[1], (_Float16)t1[2], (_Float16)t1[3]};
}
__device__ __forceinline__ void split_perm(f32x4 t0, f32x4 t1, f16x8& hi, f16x8& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = (_Float16)t0[i];
    lo[i] = (_Float16)(t0[i] - (float)hi[i]);
    hi[4 + i] = (_Float16)t1[i];
    lo[4 + i] = (_Float16)(t1[i] - (float)hi[4 + i]);
  }
}

// ---- LDS layout -------------------------------------------------------------
template <int D>
struct Lds {
  static constexpr int LDQ = D + 8;   // row stride of [64][D] fp16 arrays
  static constexpr int LDT = C + 8;   // row stride of [D][64] / [64][64] fp16 arrays
  static constexpr int LDTT = C + 16; // row stride of T~ hi/lo: 160 bytes, so the
                                      // 16-byte operand reads of 16 rows hit distinct banks
  static constexpr int LDL = C + 4;   // row stride of the fp32 64x64 L / inverse
  static constexpr int LDG = D + 4;   // row stride of per-key G [64][D] fp32
  // persistent through a chunk
  static constexpr int OFF_QT = 0;                                  // Q~   [64][LDQ] f16
  static constexpr int OFF_KHT = OFF_QT + C * LDQ * 2;              // K^ T [D][LDT] f16
  static constexpr int OFF_KTT = OFF_KHT + D * LDT * 2;             // K~ T [D][LDT] f16
  static constexpr int OFF_B = OFF_KTT + D * LDT * 2;               // B    [64][LDT] f16
  static constexpr int OFF_L = OFF_B + C * LDT * 2;                 // L/A  [64][LDL] f32
  static constexpr int OFF_SMALL = OFF_L + C * LDL * 4;
  // small arrays: G_n[D], 2^G_n[D], beta[64], scalar G[64], scan partials[4][D]
  static constexpr int SMALL_BYTES = (2 * D + 2 * C + 4 * D) * 4;
  static constexpr int OFF_A = OFF_SMALL + SMALL_BYTES;             // region A (aliased)
  // region A, phase P1..P3: G [64][LDG] f32 (per-key), raw K, raw Q: bf16 inputs
  // as staged rows [64][D] bf16 (chunk-permuted, see raw_swz; staged during the
  // previous chunk's P6, when region A holds only W), fp32 inputs as [64][LDQ] fp16
  static constexpr int A_G = 0;
  static constexpr int A_RK = A_G + C * LDG * 4;
  static constexpr int A_RQ = A_RK + C * LDQ * 2;
  static constexpr int A_END1 = A_RQ + C * LDQ * 2;
  // region A, phase P4..P6: W [64][LDQ] f16, T~ hi/lo [64][LDTT] f16, V^T [D][LDT] f16
  static constexpr int A_W = 0;
  static constexpr int A_TH = A_W + C * LDQ * 2;
  static constexpr int A_TL = A_TH + C * LDTT * 2;
  static constexpr int A_VT = A_TL + C * LDTT * 2;
  static constexpr int A_END2 = A_VT + D * LDT * 2;
  static constexpr int A_BYTES = A_END1 > A_END2 ? A_END1 : A_END2;
  static_assert(A_RK >= A_W + C * LDQ * 2, "raw K/Q staging (during P6) must not touch W");
  static_assert(C * D * 2 <= C * LDQ * 2, "a staged raw [64][D] bf16 block fits its region");
  static constexpr int TOTAL = OFF_A + A_BYTES;
  // fused back end (pass 3 only): each wavefront's share of a row's sum of
  // squares [64][up to 8] f32 (then 64 floats the lanes without a share
  // write), norm_w [D]
  static constexpr int OFF_EPI = TOTAL;
  static constexpr int OFF_ENW = OFF_EPI + (8 * C + 64) * 4;
  static constexpr int TOTAL_EPI = OFF_ENW + D * 4;
};

// What pass 3 writes per token: o (fp32), or the layer output after the
// fused back end in bf16 or fp32
enum { EPI_O = 0, EPI_BF16 = 1, EPI_F32 = 2 };
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <bool BF16>
struct RawGroup;  // 8 consecutive q/k/v elements of one token
template <>
struct RawGroup<true> { uint4 w; };
template <>
struct RawGroup<false> { f32x4 a, b; };

// `base` is uniform over the workgroup (scalar registers); `off` is the lane's
// 32-bit element offset from it, so loads use the scalar-base addressing form.
template <bool BF16>
__device__ __forceinline__ RawGroup<BF16> load_group(const void* base, uint32_t off) {
  RawGroup<BF16> r;
  if constexpr (BF16) {
    r.w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
  } else {
    const float* p = static_cast<const float*>(base) + off;
    r.a = *reinterpret_cast<const f32x4*>(p);
    r.b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  return r;
}
template <bool BF16>
__device__ __forceinline__ void unpack_group(const RawGroup<BF16>& r, float (&x)[8]) {
  if constexpr (BF16) {
    const uint32_t w[4] = {r.w.x, r.w.y, r.w.z, r.w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
      x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = r.a[i];
      x[4 + i] = r.b[i];
    }
  }
}

// Wavefronts per workgroup: one 16-row state slice per wavefront at d = 128
// (two wavefronts per SIMD), two slices per wavefront at d = 64 (one per SIMD).
template <int D>
constexpr int waves_for() { return D == 128 ? 8 : 4; }

// bf16 inputs: raw rows of a chunk go straight from HBM into LDS
// (global_load_lds_dwordx4: lane l's 16 bytes land at base + 16 l), into
// buffers that are dead during the state passing, so the prefetch of the
// next chunk holds no registers. Rows past the chunk end are loaded from row
// 0 and zeroed when they are read. `src` is the workgroup-uniform chunk base.
// This form (rows in order) stages v in the map pass; q and k use the
// chunk-permuted form below.
template <int D, int NW>
__device__ __forceinline__ void stage_rows_lds(const uint16_t* src, uint32_t HD, int n, void* lds,
                                               int wave, int lane) {
  constexpr int LPR = D / 8;                 // lanes per row (16 bytes each)
  constexpr int RPI = 64 / LPR;              // rows per wavefront instruction (1 KiB)
  constexpr int INSTR = C / RPI;             // instructions per chunk
  static_assert(INSTR % NW == 0, "every wavefront issues the same number of rows");
#pragma unroll
  for (int j = 0; j < INSTR / NW; ++j) {
    const int i = wave + NW * j;
    const int row = i * RPI + lane / LPR;
    const uint16_t* gp = src + (uint32_t)(row < n ? row : 0) * HD + 8 * (lane % LPR);
    __builtin_amdgcn_global_load_lds((gvoid_t*)gp, (lvoid_t*)(static_cast<char*>(lds) + 1024 * i),
                                     16, 0, 0);
  }
}

// Chunk permutation of the staged raw q and k rows: LDS chunk p (16 bytes) of
// row r holds chunk p ^ raw_swz<D>(r) of the row, so that sixteen consecutive
// rows read at one chunk index (the Gram operand reads) fall on distinct banks.
template <int D>
__device__ __forceinline__ int raw_swz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }

// stage_rows_lds with that permutation (lane l of an instruction still writes
// base + 16 l; it fetches the matching chunk of its row).
template <int D, int NW>
__device__ __forceinline__ void stage_rows_lds_swz(const uint16_t* src, uint32_t HD, int n, void* lds,
                                                   int wave, int lane) {
  constexpr int LPR = D / 8;
  constexpr int RPI = 64 / LPR;
  constexpr int INSTR = C / RPI;
  static_assert(INSTR % NW == 0, "every wavefront issues the same number of rows");
#pragma unroll
  for (int j = 0; j < INSTR / NW; ++j) {
    const int i = wave + NW * j;
    const int row = i * RPI + lane / LPR;
    const int chunk = (lane % LPR) ^ raw_swz<D>(row);
    const uint16_t* gp = src + (uint32_t)(row < n ? row : 0) * HD + 8 * chunk;
    __builtin_amdgcn_global_load_lds((gvoid_t*)gp, (lvoid_t*)(static_cast<char*>(lds) + 1024 * i),
                                     16, 0, 0);
  }
}

// Elements 8ch .. 8ch+7 of staged raw row r (bf16 bits), zero for rows past
// the chunk end (they hold a copy of row 0).
template <int D>
__device__ __forceinline__ uint4 raw_chunk(const unsigned char* base, int r, int ch, bool live) {
  // unconditional load, then a mask (a conditional load would toggle exec)
  const uint4 w = *reinterpret_cast<const uint4*>(base + (r * D + 8 * (ch ^ raw_swz<D>(r))) * 2);
  const uint32_t m = live ? 0xFFFFFFFFu : 0u;
  return uint4{w.x & m, w.y & m, w.z & m, w.w & m};
}
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 w) { return __builtin_bit_cast(bf16x8, w); }
__device__ __forceinline__ void bf16x8_to_f32(uint4 w, float (&x)[8]) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = bf16_bits_to_f32(u[e] & 0xFFFFu);
    x[2 * e + 1] = bf16_bits_to_f32(u[e] >> 16);
  }
}

// hi + lo bf16 split of eight values, two per conversion: hi rounds to
// nearest, lo is the rounded remainder (hi + lo carries about 16 bits).
__device__ __forceinline__ void split8_bf16(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  uint32_t h[4], l[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const bf16x2 hp = __builtin_convertvector(f32x2{x[2 * p], x[2 * p + 1]}, bf16x2);
    const uint32_t hb = __builtin_bit_cast(uint32_t, hp);
    const float r0 = x[2 * p] - __uint_as_float(hb << 16);
    const float r1 = x[2 * p + 1] - __uint_as_float(hb & 0xFFFF0000u);
    h[p] = hb;
    l[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r0, r1}, bf16x2));
  }
  hi = __builtin_bit_cast(bf16x8, uint4{h[0], h[1], h[2], h[3]});
  lo = __builtin_bit_cast(bf16x8, uint4{l[0], l[1], l[2], l[3]});
}

// A contiguous block of n_kib KiB from HBM into LDS, one KiB per wavefront
// instruction (lane l moves bytes 16 l .. 16 l + 15 of it).
template <int NW>
__device__ __forceinline__ void stage_block_lds(const void* src, int n_kib, void* lds, int wave, int lane) {
  for (int i = wave; i < n_kib; i += NW)
    __builtin_amdgcn_global_load_lds((gvoid_t*)(static_cast<const char*>(src) + 1024 * i + 16 * lane),
                                     (lvoid_t*)(static_cast<char*>(lds) + 1024 * i), 16, 0, 0);
}

// Registers holding one chunk's raw inputs (prefetched during the previous chunk).
template <int D, bool BF16, bool PER_KEY, int NT>
struct ChunkRegs {
  static constexpr int GROUPS = C * D / 8;       // 8-element groups per [64][D] tensor
  static constexpr int GPT = GROUPS / NT;        // groups per thread
  static constexpr int TPB = C * D / NT;         // per-key alpha: tokens per thread
  RawGroup<BF16> k[BF16 ? 1 : GPT], q[BF16 ? 1 : GPT], v[GPT];   // bf16: q, k staged in LDS
  // per-key: channel tid % D, tokens TPB (tid / D) .. +TPB-1; scalar: token = lane (wave 0)
  float alpha[PER_KEY ? TPB : 1];
  float beta;
};

// Every address is a workgroup-uniform base (scalar registers, cheap to
// recompute per access) plus a 32-bit per-lane offset.
// h is the value head (v, o and the state); q, k, alpha and beta belong to head
// h >> qk_shift of a.H >> qk_shift (qk_shift = 1: d_v = 2 d_k, each head's state
// rows split into two value heads of d_k rows that share q, k and the gates).
//
// Rows (v; fp32 q and k) of one chunk into registers.
template <int D, bool BF16, bool PER_KEY, int NT>
__device__ __forceinline__ void load_chunk_rows(ChunkRegs<D, BF16, PER_KEY, NT>& R, const PrefillArgs& a,
                                                int64_t tok0, int n, int h, int tid, bool load_v) {
  // Every load is unconditional: rows and tokens past the chunk's n (>= 1)
  // read row n - 1 again, and their values are masked where they are used
  // (unpack_masked, the decay scan, beta). A load under a lane mask, or a
  // select right after one, costs a branch per load and can make the compiler
  // wait for every load in flight.
  using CR = ChunkRegs<D, BF16, PER_KEY, NT>;
  constexpr int ROWS_PER_PASS = NT / (D / 8);     // tokens covered by one group pass
  const int Hq = a.H >> a.qk_shift, hq = h >> a.qk_shift;
  const uint32_t HD = (uint32_t)a.H * D;          // v elements per token (all heads)
  const uint32_t HDq = (uint32_t)Hq * D;          // q/k/alpha elements per token
  const int64_t row0 = (tok0 * a.H + h) * D;      // first v element of this chunk and head
  const int64_t rowq0 = (tok0 * Hq + hq) * D;     // first q/k element
  const int c0 = tid / (D / 8), k8 = tid % (D / 8);
  const int last = n - 1;
#pragma unroll
  for (int j = 0; j < CR::GPT; ++j) {
    const uint32_t c = (uint32_t)min(c0 + j * ROWS_PER_PASS, last);
    const uint32_t off = c * HD + 8u * k8, offq = c * HDq + 8u * k8;
    if constexpr (BF16) {
      if (load_v) R.v[j] = load_group<true>(static_cast<const uint16_t*>(a.v) + row0, off);
    } else {
      R.k[j] = load_group<false>(static_cast<const float*>(a.k) + rowq0, offq);
      R.q[j] = load_group<false>(static_cast<const float*>(a.q) + rowq0, offq);
      if (load_v) R.v[j] = load_group<false>(static_cast<const float*>(a.v) + row0, off);
    }
  }
}
// alpha and beta of one chunk into registers (unconditional, as above).
template <int D, bool BF16, bool PER_KEY, int NT>
__device__ __forceinline__ void load_chunk_gates(ChunkRegs<D, BF16, PER_KEY, NT>& R, const PrefillArgs& a,
                                                 int64_t tok0, int n, int h, int tid) {
  using CR = ChunkRegs<D, BF16, PER_KEY, NT>;
  const int Hq = a.H >> a.qk_shift, hq = h >> a.qk_shift;
  const uint32_t HDq = (uint32_t)Hq * D;
  const int64_t rowq0 = (tok0 * Hq + hq) * D;
  const int last = n - 1;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), lane = tid % 64;
  if constexpr (PER_KEY) {
    const int kcol = tid % D, cb = tid / D;
#pragma unroll
    for (int j = 0; j < CR::TPB; ++j) {
      const uint32_t c = (uint32_t)min(CR::TPB * cb + j, last);
      R.alpha[j] = a.alpha[rowq0 + c * HDq + kcol];
    }
  } else {
    R.alpha[0] = wave == 0 ? a.alpha[(tok0 + min(lane, last)) * Hq + hq] : 1.f;
  }
  R.beta = wave == 0 ? a.beta[(tok0 + min(lane, last)) * Hq + hq] : 0.f;
}
// Both parts of a chunk's register inputs.
template <int D, bool BF16, bool PER_KEY, int NT>
__device__ __forceinline__ void load_chunk(ChunkRegs<D, BF16, PER_KEY, NT>& R, const PrefillArgs& a,
                                           int64_t tok0, int n, int h, int tid, bool load_v) {
  load_chunk_rows<D, BF16, PER_KEY, NT>(R, a, tok0, n, h, tid, load_v);
  load_chunk_gates<D, BF16, PER_KEY, NT>(R, a, tok0, n, h, tid);
}

// Gram tile pairs (R, I), R >= I, as runs of one row block per wavefront:
// run `run` of wavefront `wave` covers (R, I0..I1); false when it has none.
// A wavefront whose runs end on diagonal pairs then inverts those diagonal
// blocks (gram_diag). Balance counts a pair and an inversion as one unit
// each, per SIMD:
//   four wavefronts:  w0: R3 I0-2 | w1: R2 I0-1, R1 I0 | w2: R0 I0, R1 I1, inv 0,1
//                     | w3: R2 I2, R3 I3, inv 2,3                       (3/3/3/3)
//   eight wavefronts (w and w+4 share a SIMD), scalar gate (cheap pairs):
//                     wavefront b < 4 computes the diagonal pair (b, b) and
//                     inverts block b, so only one pair precedes each
//                     inversion; w4: R3 I0-1 | w5: R3 I2, R2 I1 | w6: R2 I0 |
//                     w7: R1 I0. Per-key gate (a pair costs more than an
//                     inversion, and the pairs of a run share their row
//                     operands): w0: R3 I0-1 | w1: R3 I2-3, inv 3 | w2: R2 I0 |
//                     w3: R2 I2, inv 2 | w4: R1 I0 | w5: R2 I1 | w6: R0 I0,
//                     inv 0 | w7: R1 I1, inv 1 (per SIMD two row operands, at
//                     most three pairs and one or two inversions)
// Four 12-bit run codes in the 16-bit fields of one 64-bit constant (field w
// for wavefront w): the lookup is register arithmetic, not a memory load.
constexpr uint64_t pack_runs(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  return (uint64_t)w0 | ((uint64_t)w1 << 16) | ((uint64_t)w2 << 32) | ((uint64_t)w3 << 48);
}
template <int NW, bool PER_KEY>
__device__ __forceinline__ bool gram_run(int wave_lane, int run, int& R, int& I0, int& I1) {
  // per wavefront and run a nibble triple (R, I0, I1); 0xFFF = no run. The
  // wavefront index is uniform: the selection runs on scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(wave_lane);
  uint64_t packed;
  if constexpr (NW == 4) {
    constexpr uint64_t kRun0 = pack_runs(0x302, 0x201, 0x000, 0x222);
    constexpr uint64_t kRun1 = pack_runs(0xFFF, 0x100, 0x111, 0x333);
    packed = run == 0 ? kRun0 : kRun1;
  } else {
    static_assert(NW == 8, "four or eight wavefronts");
    constexpr uint64_t kRun0Lo = !PER_KEY ? pack_runs(0x000, 0x111, 0x222, 0x333)    // wavefronts 0-3
                                          : pack_runs(0x301, 0x323, 0x200, 0x222);
    constexpr uint64_t kRun0Hi = !PER_KEY ? pack_runs(0x301, 0x322, 0x200, 0x100)    // wavefronts 4-7
                                          : pack_runs(0x100, 0x211, 0x000, 0x111);
    constexpr uint64_t kRun1Lo = pack_runs(0xFFF, 0xFFF, 0xFFF, 0xFFF);
    constexpr uint64_t kRun1Hi = !PER_KEY ? pack_runs(0xFFF, 0x211, 0xFFF, 0xFFF)
                                          : pack_runs(0xFFF, 0xFFF, 0xFFF, 0xFFF);
    const bool hi = (wave & 7) >= 4;
    packed = run == 0 ? (hi ? kRun0Hi : kRun0Lo) : (hi ? kRun1Hi : kRun1Lo);
  }
  const uint32_t code = (uint32_t)(packed >> (16 * (wave & 3))) & 0xFFFu;
  if (code == 0xFFF) return false;
  R = code >> 8;
  I0 = (code >> 4) & 15;
  I1 = code & 15;
  return true;
}
// Diagonal blocks this wavefront inverts after its runs (d0, d1; equal when it
// inverts one block), or false.
template <int NW, bool PER_KEY>
__device__ __forceinline__ bool gram_diag(int wave, int& d0, int& d1) {
  if constexpr (NW == 4) {
    if (wave == 2) { d0 = 0; d1 = 1; return true; }
    if (wave == 3) { d0 = 2; d1 = 3; return true; }
    return false;
  } else if constexpr (PER_KEY) {
    // the wavefront whose run ends on the diagonal pair (b, b) inverts block b
    const int b = wave == 6 ? 0 : wave == 7 ? 1 : wave == 3 ? 2 : wave == 1 ? 3 : -1;
    d0 = d1 = b;
    return b >= 0;
  } else {
    if (wave < 4) { d0 = wave; d1 = wave; return true; }
    return false;
  }
}

// Two fp32 accumulator tiles (t1 may be zero) as hi + lo bf16 permuted-K
// operands: hi rounds to nearest, lo is the rounded remainder.
__device__ __forceinline__ void split_tiles_bf16(f32x4 t0, f32x4 t1, bf16x8& hi, bf16x8& lo) {
  const float x[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
  split8_bf16(x, hi, lo);
}
// T~ rows 16R + 4g + i, column col of one accumulator tile (lane (g, l16)),
// scaled by beta_col, as fp16 hi + lo.
template <class L>
__device__ __forceinline__ void put_t_tile(_Float16* sTh, _Float16* sTl, f32x4 a, float b, int row0, int col) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float t = a[i] * b;
    const _Float16 th = (_Float16)t;
    sTh[(row0 + i) * L::LDTT + col] = th;
    sTl[(row0 + i) * L::LDTT + col] = (_Float16)(t - (float)th);
  }
}

// Off-diagonal blocks of block column I of A = (I + L)^-1 (sL holds L below
// the diagonal blocks and A_RR on them, fp32 row-major): one wavefront, on
// fp32 MFMA (16x16x4, no operand conversion). The column's tiles stay in
// accumulator layout (lane (g, l16): rows 4g+i, column l16) and enter the
// next products as the permuted-K operand (K-step s: lane group g supplies
// k = 4g + s), against rows of L and A_RR read in the same order, all of
// them read before the chain starts.
template <int I, class L>
__device__ __forceinline__ void inverse_column(const float* sL, const float* sBeta, _Float16* sTh, _Float16* sTl,
                                               int lane) {
  const int g = lane >> 4, l16 = lane & 15;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 Acol[4], lrow[4][3], drow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) Acol[I][i] = sL[(16 * I + 4 * g + i) * L::LDL + 16 * I + l16];
#pragma unroll
  for (int R = I + 1; R < 4; ++R) {
    const float* lr = sL + (16 * R + l16) * L::LDL;
#pragma unroll
    for (int m = I; m < R; ++m) lrow[R][m - I] = *reinterpret_cast<const f32x4*>(lr + 16 * m + 4 * g);
    drow[R] = *reinterpret_cast<const f32x4*>(lr + 16 * R + 4 * g);
  }
  const float bcol = sBeta[16 * I + l16];
#pragma unroll
  for (int R = I + 1; R < 4; ++R) {
    // acc = sum_{m=I}^{R-1} L_Rm A_mI
    f32x4 acc = zero;
#pragma unroll
    for (int m = I; m < R; ++m)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mfma_f32(lrow[R][m - I][ks], Acol[m][ks], acc);
    // A_RI = -A_RR acc
    f32x4 res = zero;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) res = mfma_f32(drow[R][ks], acc[ks], res);
#pragma unroll
    for (int i = 0; i < 4; ++i) Acol[R][i] = -res[i];
  }
  // T~_RI = A_RI Diag(beta), written once the chain is done
#pragma unroll
  for (int R = I + 1; R < 4; ++R) put_t_tile<L>(sTh, sTl, Acol[R], bcol, 16 * R + 4 * g, 16 * I + l16);
}

// The rest of T~ for wavefront w of the NW - 3 that run no column chain: the
// diagonal blocks A_RR Diag(beta) (R = w, w + NW - 3, ..) and, on the last of
// those wavefronts, zeros above the diagonal.
template <int NW, class L>
__device__ __forceinline__ void inverse_rest(const float* sL, const float* sBeta, _Float16* sTh, _Float16* sTl, int w,
                                             int lane) {
  constexpr int NR = NW - 3;
  const int row = lane >> 2, c4 = 4 * (lane & 3);     // 16 rows x 4 column groups of 4
#pragma unroll
  for (int R = 0; R < 4; ++R) {
    if (R % NR != w) continue;
    const f32x4 a = *reinterpret_cast<const f32x4*>(sL + (16 * R + row) * L::LDL + 16 * R + c4);
    const f32x4 b = *reinterpret_cast<const f32x4*>(sBeta + 16 * R + c4);
    f16x4 th, tl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float t = a[e] * b[e];
      th[e] = (_Float16)t;
      tl[e] = (_Float16)(t - (float)th[e]);
    }
    *reinterpret_cast<f16x4*>(sTh + (16 * R + row) * L::LDTT + 16 * R + c4) = th;
    *reinterpret_cast<f16x4*>(sTl + (16 * R + row) * L::LDTT + 16 * R + c4) = tl;
  }
  if (w == NR - 1) {
    // blocks (R, I), I > R: 6 blocks x 16 rows x 16 columns, 8 halves per piece
    const f16x8 z = {};
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int p = lane + 64 * j;                     // 192 pieces of 8 halves
      const int blk = p / 32, r = (p % 32) / 2, half = p % 2;
      const int R = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
      const int I = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
      const int off = (16 * R + r) * L::LDTT + 16 * I + 8 * half;
      *reinterpret_cast<f16x8*>(sTh + off) = z;
      *reinterpret_cast<f16x8*>(sTl + off) = z;
    }
  }
}

__device__ __forceinline__ float wave_inclusive_scan(float x, int lane) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const float y = __shfl_up(x, m);
    if (lane >= m) x += y;
  }
  return x;
}

template <int D, bool BF16, bool PER_KEY, bool MAP, bool WU, int NW, int EPI = EPI_O>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void prefill_kernel(PrefillArgs a) {
  static_assert(!(MAP && WU), "the map pass forms W and U' itself");
  static_assert(EPI == EPI_O || (WU && BF16), "the fused back end runs in pass 3 of bf16 inputs");
  constexpr int NT = 64 * NW;    // threads
  using L = Lds<D>;
  using CR = ChunkRegs<D, BF16, PER_KEY, NT>;
  constexpr int SPW = D / (16 * NW);   // state slices per wavefront
  static_assert(SPW >= 1 && SPW * 16 * NW == D, "slices cover the state");
  static_assert(NT / D >= 1 && NT / D <= 4, "per-key scan partials: at most four blocks of tokens");
  constexpr int NSL = MAP ? 2 * SPW : SPW;   // MAP: SPW N slices, then SPW M slices
  constexpr int KT = D / 16;     // 16-row tiles along d_k
  extern __shared__ __align__(16) unsigned char smem[];

  _Float16* sQt = reinterpret_cast<_Float16*>(smem + L::OFF_QT);
  _Float16* sKhT = reinterpret_cast<_Float16*>(smem + L::OFF_KHT);
  _Float16* sKtT = reinterpret_cast<_Float16*>(smem + L::OFF_KTT);
  _Float16* sB = reinterpret_cast<_Float16*>(smem + L::OFF_B);
  float* sL = reinterpret_cast<float*>(smem + L::OFF_L);
  float* sGL = reinterpret_cast<float*>(smem + L::OFF_SMALL);   // [D] G_n per channel
  float* sGam = sGL + D;                                          // [D] 2^G_n
  float* sBeta = sGam + D;                                        // [64]
  float* sGs = sBeta + C;                                         // [64] scalar-gate G
  float* sPart = sGs + C;                                         // [4][D] cumsum partials
  float* sDec = sPart;         // scalar gate (sPart unused): [64] 2^G_c, then [64] 2^(G_n - G_c)
  float* sRem = sPart + C;
  unsigned char* regA = smem + L::OFF_A;
  float* sG = reinterpret_cast<float*>(regA + L::A_G);
  [[maybe_unused]] float* sEP = reinterpret_cast<float*>(smem + L::OFF_EPI);
  [[maybe_unused]] float* sENw = reinterpret_cast<float*>(smem + L::OFF_ENW);
  _Float16* sRK = reinterpret_cast<_Float16*>(regA + L::A_RK);
  _Float16* sRQ = reinterpret_cast<_Float16*>(regA + L::A_RQ);
  // WU: the stored W is loaded into the L buffer (no inverse is formed there)
  _Float16* sW = reinterpret_cast<_Float16*>(WU ? smem + L::OFF_L : regA + L::A_W);
  _Float16* sTh = reinterpret_cast<_Float16*>(regA + L::A_TH);
  _Float16* sTl = reinterpret_cast<_Float16*>(regA + L::A_TL);
  _Float16* sVT = reinterpret_cast<_Float16*>(regA + L::A_VT);

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int g = lane >> 4, l16 = lane & 15;
  const int item_idx = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const PrefillItem item = work_item(a, item_idx);
  if constexpr (MAP || WU) {
    // every segment of a split sequence: the maps of all but the last feed the
    // scan, and each chunk's W and U' are kept for pass 3 (WU)
    if (item.n_segs <= 1) return;                // (uniform)
  } else {
    if (item.n_segs > 1) return;                 // split sequences run in WU
  }
  constexpr bool out_mode = !MAP;
  // MAP with bf16 inputs stages v rows in LDS as well (into the Q~ buffer,
  // which MAP never uses), so its prefetch holds no registers across P6
  constexpr bool v_in_lds = MAP && BF16;
  constexpr bool v_in_regs = !v_in_lds && !WU;   // WU reads no v (U' is stored)
  // Pass 3 of a split sequence's segment (WU): the map pass already formed each
  // chunk's W and U' (P5) and stored them; they are loaded instead of being
  // formed again from the inverse (same arithmetic, same bits). The stored W is
  // the LDS image of the W buffer, 1 KiB per wavefront load.
  constexpr int W_BYTES = (int)wu_w_bytes(D);
  static_assert(W_BYTES == C * L::LDQ * 2 && W_BYTES % 1024 == 0 && W_BYTES <= C * L::LDL * 4,
                "stored W layout");
  constexpr int64_t WU_BYTES = (int64_t)wu_chunk_bytes(D);
  unsigned char* wu_base = nullptr;
  if constexpr (MAP || WU)
    wu_base = static_cast<unsigned char*>(a.seg_wu) + ((int64_t)item_idx * a.H + h) * a.seg_chunks * WU_BYTES;
  const int64_t HD = (int64_t)a.H * D;
  const int64_t DD = (int64_t)D * D;

  // ---- start state: S0^T in accumulator layout ------------------------------
  // slice sl of this wavefront covers state rows 16 (SPW wave + sl % SPW) .. +15
  // (MAP: sl < SPW are N rows, sl >= SPW the same rows of M);
  // tile kt, lane l: S0^T[k = 16kt + 4g + i][v = 16 slice + l16] = S0[v][k]
  f32x4 ST[NSL][KT];
  {
    const float* src = nullptr;
    if constexpr (!MAP) {
      // a split sequence takes every start state, S_0 included, from the scan,
      // so this pass never reads initial_state (which may alias final_state,
      // written by the sequence's last segment)
      if (item.n_segs > 1) src = a.seg_states + ((int64_t)item_idx * a.H + h) * DD;
      else if (a.init) src = a.init + ((int64_t)item.seq * a.H + h) * DD;
    }
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      const int row = 16 * (SPW * wave + sl % SPW) + l16;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        if (src) {
          ST[sl][kt] = *reinterpret_cast<const f32x4*>(src + row * D + 16 * kt + 4 * g);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            ST[sl][kt][i] = (MAP && sl >= SPW && row == 16 * kt + 4 * g + i) ? 1.f : 0.f;
        }
      }
    }
  }
  // vmcnt(0): the start state has landed. Without this wait on every path into
  // the chunk loop, the compiler keeps the load pending around the loop and
  // waits for all vector memory traffic (the next chunk's prefetch included)
  // before the state's first use in every chunk.
  __builtin_amdgcn_s_waitcnt(0x0F70);

  const int n_chunks = (item.n_tokens + C - 1) / C;
  const uint32_t HDu = (uint32_t)a.H * D;                       // v row stride (elements)
  const int Hq = a.H >> a.qk_shift, hq = h >> a.qk_shift;       // q/k head (see load_chunk)
  const uint32_t HDqu = (uint32_t)Hq * D;                       // q/k row stride
  if constexpr (EPI != EPI_O)
    for (int e = tid; e < D; e += NT) sENw[e] = a.norm_w[e];    // read after the barriers below
  CR regs;
  // Per-key gate: the local part of a chunk's decay scan (thread: channel
  // tid % D, tokens TPB cb .. TPB cb + TPB-1) runs before the chunk starts
  // (for chunk c + 1 at the end of chunk c, on its prefetched alpha), with
  // the block totals in sPart, so P1 combines them behind one barrier.
  float gloc[PER_KEY ? CR::TPB : 1];
  [[maybe_unused]] auto local_scan = [&](int n_) __attribute__((always_inline)) {
    const int kcol = tid % D, cb = tid / D;
    float run = 0.f;
#pragma unroll
    for (int j = 0; j < CR::TPB; ++j) {
      run += log2_hw(CR::TPB * cb + j < n_ ? regs.alpha[j] : 1.f);
      gloc[j] = run;
    }
    sPart[cb * D + kcol] = run;
  };
  if (n_chunks > 0) {
    load_chunk<D, BF16, PER_KEY, NT>(regs, a, item.tok_begin, min(C, item.n_tokens), h, tid, v_in_regs);
    if constexpr (BF16) {
      const int64_t row0 = (item.tok_begin * a.H + h) * D;
      const int64_t rowq0 = (item.tok_begin * Hq + hq) * D;
      if constexpr (v_in_lds)
        stage_rows_lds<D, NW>(static_cast<const uint16_t*>(a.v) + row0, HDu, min(C, item.n_tokens),
                          smem + L::OFF_QT, wave, lane);
      stage_rows_lds_swz<D, NW>(static_cast<const uint16_t*>(a.k) + rowq0, HDqu, min(C, item.n_tokens),
                                regA + L::A_RK, wave, lane);
      if constexpr (!MAP)
        stage_rows_lds_swz<D, NW>(static_cast<const uint16_t*>(a.q) + rowq0, HDqu, min(C, item.n_tokens),
                                  regA + L::A_RQ, wave, lane);
    }
    if constexpr (PER_KEY) local_scan(min(C, item.n_tokens));
    if constexpr (BF16) __builtin_amdgcn_s_waitcnt(0);   // staged rows have landed in LDS
    __syncthreads();
  }

  // Fused back end (pass 3 of the KDA layer): a chunk's O tiles and output-gate
  // logits are held until the next chunk starts, when every wavefront's share
  // of each row's sum of squares is in LDS; one 16-token tile ct of a chunk
  // whose outputs start at element eb and hold n_ tokens (rows at or past n_
  // go to the sink): out = o rsqrt(mean o^2 + eps) norm_w sigmoid(g). The
  // shares combine pairwise in wavefront order, the order in which the
  // separate back-end kernel's xor shuffles combine its lanes (same bits).
  [[maybe_unused]] f32x4 Oh[EPI != EPI_O ? 4 : 1] = {};   // (the first chunk's back end reads them:
  [[maybe_unused]] u32x2 gh[EPI != EPI_O ? 4 : 1] = {};   // its stores go to the sink)
  [[maybe_unused]] auto epi_tile = [&](int ct, int64_t eb, int n_, int g_, int l16_) __attribute__((always_inline)) {
    const int c = 16 * ct + l16_;
    float ss;
    if constexpr (NW == 4) {
      const f32x4 pp = *reinterpret_cast<const f32x4*>(sEP + 4 * c);
      ss = (pp[0] + pp[1]) + (pp[2] + pp[3]);
    } else {
      const f32x4 p0 = *reinterpret_cast<const f32x4*>(sEP + 8 * c);
      const f32x4 p1 = *reinterpret_cast<const f32x4*>(sEP + 8 * c + 4);
      ss = ((p0[0] + p0[1]) + (p0[2] + p0[3])) + ((p1[0] + p1[1]) + (p1[2] + p1[3]));
    }
    const float r = __builtin_amdgcn_rsqf(ss / D + a.eps);
    const int w_ = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const f32x4 w4 = *reinterpret_cast<const f32x4*>(sENw + 16 * w_ + 4 * g_);
    const u32x2 gb = gh[ct];
    const float gv[4] = {bf16_bits_to_f32(gb[0] & 0xFFFFu), bf16_bits_to_f32(gb[0] >> 16),
                         bf16_bits_to_f32(gb[1] & 0xFFFFu), bf16_bits_to_f32(gb[1] >> 16)};
    f32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = Oh[ct][e] * r * w4[e] * sigmoid_rcp(gv[e]);
    // unconditional stores (rows past the end go to the sink): a store under
    // a lane mask makes later waits for loads drain these stores
    const int64_t off = eb + (int64_t)c * HD;
    if constexpr (EPI == EPI_BF16) {
      uint16_t* dst = c < n_ ? static_cast<uint16_t*>(a.out) + off : static_cast<uint16_t*>(a.out_sink);
      *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
    } else {
      float* dst = c < n_ ? static_cast<float*>(a.out) + off : static_cast<float*>(a.out_sink);
      *reinterpret_cast<f32x4*>(dst) = y;
    }
  };

  for (int ch = 0; ch < n_chunks; ++ch) {
    const int64_t tok0 = item.tok_begin + (int64_t)ch * C;
    const int n = min(C, item.n_tokens - ch * C);
    // Per-lane index arithmetic is redone every chunk: hoisted out of the
    // loop it would hold dozens of registers for the whole item.
    int tid_c = tid;
    asm volatile("" : "+v"(tid_c));
    const int tid = tid_c, lane = tid_c % 64, g = lane >> 4, l16 = lane & 15;

    // U' = T~ V for this wavefront's value slices (rows c in 4 tiles): formed in
    // P5, or (WU) the stored one, fetched here with W. W goes through registers
    // and is written to LDS after P3: an LDS-bound load issued here would make
    // the LDS reads of P1-P3 wait for it.
    f32x4 Up[SPW][4];
    constexpr int W_VEC = W_BYTES / 16;               // 16-byte pieces of W
    constexpr int W_PER_T = (W_VEC + NT - 1) / NT;
    f32x4 wreg[WU ? W_PER_T : 1];
    if constexpr (WU) {
      const unsigned char* rec = wu_base + (int64_t)ch * WU_BYTES;
#pragma unroll
      for (int j = 0; j < W_PER_T; ++j) {
        const int e = tid + j * NT;
        if (e < W_VEC) wreg[j] = reinterpret_cast<const f32x4*>(rec)[e];
      }
      const f32x4* up = reinterpret_cast<const f32x4*>(rec + W_BYTES);
#pragma unroll
      for (int sl = 0; sl < SPW; ++sl)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) Up[sl][ct] = up[((SPW * wave + sl) * 4 + ct) * 64 + lane];
    }
    if constexpr (EPI != EPI_O) {
      // this chunk's output-gate logits (rows past the end read the last
      // row), then the back end of the previous chunk (a full one; at the
      // first chunk every row goes to the sink)
      const int64_t eb = tok0 * HD + (int64_t)h * D + 16 * wave + 4 * g;
      u32x2 gn[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        gn[ct] = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.g_logit) + eb +
                                                 (int64_t)min(16 * ct + l16, n - 1) * HD);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) epi_tile(ct, eb - C * HD, ch > 0 ? C : 0, g, l16);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) gh[ct] = gn[ct];
    }

    // ---- P1: cumulative log2 decay, beta; fp32 inputs: q, k to fp16 ---------
    // (bf16 q, k are read straight from their staged rows in P2 and P3)
    if constexpr (!BF16) {
#pragma unroll
      for (int j = 0; j < CR::GPT; ++j) {
        const int gi = tid + j * NT;
        const int c = gi / (D / 8), k8 = gi % (D / 8);
        f16x8 kh, qh;
        float x[8];
        unpack_group<BF16>(regs.k[j], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) kh[e] = (_Float16)(c < n ? x[e] : 0.f);
        unpack_group<BF16>(regs.q[j], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) qh[e] = (_Float16)(c < n ? x[e] : 0.f);
        *reinterpret_cast<f16x8*>(sRK + c * L::LDQ + 8 * k8) = kh;
        if constexpr (!MAP) *reinterpret_cast<f16x8*>(sRQ + c * L::LDQ + 8 * k8) = qh;
      }
    }
    if constexpr (PER_KEY) {
      // the local scans (gloc, sPart) ran before this chunk: combine the
      // block totals of the earlier token blocks
      const int kcol = tid % D, cb = tid / D;
      float pre = 0.f;
      for (int b = 0; b < cb; ++b) pre += sPart[b * D + kcol];
#pragma unroll
      for (int j = 0; j < CR::TPB; ++j) sG[(CR::TPB * cb + j) * L::LDG + kcol] = pre + gloc[j];
      if (cb == NT / D - 1) {
        sGL[kcol] = pre + gloc[CR::TPB - 1];
        sGam[kcol] = exp2_hw(pre + gloc[CR::TPB - 1]);
      }
    } else {
      if (wave == 0) {
        const float gcum = wave_inclusive_scan(log2_hw(lane < n ? regs.alpha[0] : 1.f), lane);
        sGs[lane] = gcum;
        const float gl = __shfl(gcum, C - 1);
        const float gam = exp2_hw(gl);
        sGL[lane] = gl;
        sGam[lane] = gam;
        sDec[lane] = exp2_hw(gcum);
        sRem[lane] = exp2_hw(gl - gcum);
        if (D > 64) { sGL[lane + 64] = gl; sGam[lane + 64] = gam; }
      }
    }
    if (wave == 0) sBeta[lane] = lane < n ? regs.beta : 0.f;
    __syncthreads();
    // The next chunk's register inputs are fetched as soon as this chunk's
    // are consumed (gates here, rows after P4), so their loads spread over the
    // chunk instead of queueing behind each other before P6. The fetches are
    // unconditional: the last chunk fetches itself again.
    const int ch_next = min(ch + 1, n_chunks - 1);
    const int64_t tok_next = item.tok_begin + (int64_t)ch_next * C;
    const int n_next = min(C, item.n_tokens - ch_next * C);
    load_chunk_gates<D, BF16, PER_KEY, NT>(regs, a, tok_next, n_next, h, tid);

    // ---- P2: decayed operands ------------------------------------------------
#pragma unroll
    for (int j = 0; j < CR::GPT; ++j) {
      const int gi = tid + j * NT;
      const int c = gi / (D / 8), k8 = gi % (D / 8);
      float kx[8], qx[8] = {};
      if constexpr (BF16) {
        bf16x8_to_f32(raw_chunk<D>(regA + L::A_RK, c, k8, c < n), kx);
        if constexpr (!MAP) bf16x8_to_f32(raw_chunk<D>(regA + L::A_RQ, c, k8, c < n), qx);
      } else {
        const f16x8 kh = *reinterpret_cast<const f16x8*>(sRK + c * L::LDQ + 8 * k8);
#pragma unroll
        for (int e = 0; e < 8; ++e) kx[e] = (float)kh[e];
        if constexpr (!MAP) {
          const f16x8 qh = *reinterpret_cast<const f16x8*>(sRQ + c * L::LDQ + 8 * k8);
#pragma unroll
          for (int e = 0; e < 8; ++e) qx[e] = (float)qh[e];
        }
      }
      f16x8 qt;
      // scalar gate: one factor pair per token, computed once in P1
      const float dec_c = PER_KEY ? 0.f : sDec[c], rem_c = PER_KEY ? 0.f : sRem[c];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = 8 * k8 + e;
        float dec = dec_c, rem = rem_c;
        if constexpr (PER_KEY) {
          const float gc = sG[c * L::LDG + kk];
          dec = exp2_hw(gc);
          rem = exp2_hw(sGL[kk] - gc);
        }
        const float kf = kx[e];
        qt[e] = (_Float16)(qx[e] * dec);
        if constexpr (!WU) sKhT[kk * L::LDT + swz(kk, c)] = (_Float16)(kf * dec);   // (W, P5)
        sKtT[kk * L::LDT + swz(kk, c)] = (_Float16)(kf * rem);
      }
      if constexpr (!MAP) *reinterpret_cast<f16x8*>(sQt + c * L::LDQ + 8 * k8) = qt;
    }

    // ---- P3: Gram tiles L (fp32) and B (fp16) ------------------------------
    // Upper blocks of B are zero. The 10 lower tile pairs (R >= I) go to the
    // wavefronts as runs (R, I0..I1) of one row block (gram_run). Each pair computes the transposed tiles L^T and B^T (column block I as the
    // A operand, row block R as the B operand), so a lane ends with four
    // consecutive columns i of one row r and stores them as one vector.
    for (int e = tid; e < (MAP ? 0 : 6 * 256); e += NT) {
      const int t = e / 256, rr = (e % 256) / 16, cc = e % 16;
      const int R = t < 3 ? 0 : (t < 5 ? 1 : 2);
      const int I = t < 3 ? t + 1 : (t < 5 ? t - 1 : 3);
      sB[(16 * R + rr) * L::LDT + 16 * I + cc] = (_Float16)0.f;
    }
    {
#pragma unroll
      for (int run = 0; run < 2; ++run) {
        int R, I0, I1;
        if (!gram_run<NW, PER_KEY>(wave, run, R, I0, I1)) break;
        const int r = 16 * R + l16;                  // this lane's row of L / B
        if constexpr (!PER_KEY) {
          // exact products of the inputs (bf16 MFMA on the staged bf16 rows, fp16
          // MFMA on the fp16 copy of fp32 inputs); decay applied per element
          using OpT = typename std::conditional<BF16, bf16x8, f16x8>::type;
          auto gram_op = [&](const unsigned char* raw, const _Float16* cp, int row0, int ks) -> OpT {
            if constexpr (BF16) {
              const int row = row0 + l16;
              return as_bf16x8(raw_chunk<D>(raw, row, 4 * ks + g, row < n));
            } else {
              return ld_std(cp, L::LDQ, row0, 32 * ks, lane);
            }
          };
          OpT kr[D / 32], qr[D / 32];
#pragma unroll
          for (int ks = 0; ks < D / 32; ++ks) {
            kr[ks] = gram_op(regA + L::A_RK, sRK, 16 * R, ks);
            if constexpr (!MAP) qr[ks] = gram_op(regA + L::A_RQ, sRQ, 16 * R, ks);
          }
          const float gr = sGs[r], br = sBeta[r];
          for (int I = I0; I <= I1; ++I) {
            f32x4 accL = {0, 0, 0, 0}, accB = {0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
              const OpT ki = gram_op(regA + L::A_RK, sRK, 16 * I, ks);
              if constexpr (BF16) {
                if constexpr (!WU) accL = mfma_bf16(ki, kr[ks], accL);
                if constexpr (!MAP) accB = mfma_bf16(ki, qr[ks], accB);
              } else {
                if constexpr (!WU) accL = mfma_f16(ki, kr[ks], accL);
                if constexpr (!MAP) accB = mfma_f16(ki, qr[ks], accB);
              }
            }
            const int i0 = 16 * I + 4 * g;           // columns i0..i0+3 of row r
            const f32x4 gi = *reinterpret_cast<const f32x4*>(sGs + i0);
            f32x4 lv;
            f16x4 bv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float f = exp2_hw(fminf(gr - gi[e], 0.f));
              lv[e] = (i0 + e < r) ? accL[e] * f * br : 0.f;
              bv[e] = (_Float16)((i0 + e <= r) ? accB[e] * f : 0.f);
            }
            if constexpr (!WU) *reinterpret_cast<f32x4*>(sL + r * L::LDL + i0) = lv;
            if constexpr (!MAP) *reinterpret_cast<f16x4*>(sB + r * L::LDT + i0) = bv;
            if (!WU && I == R) {
              // diagonal tile: L_RR^T also into its upper triangle (column i
              // of L_RR becomes row i there); issued after the row stores, so
              // it lands after their zeros
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (i0 + e < r) sL[(i0 + e) * L::LDL + r] = lv[e];
            }
          }
        } else {
          // three-term bf16 products of operands decayed relative to token 16R:
          // row side 2^(G_r - G_16R) <= 1, column side 2^(G_16R - G_i) (<= 1
          // for i <= 16R, bounded inside block R). L and B share the column
          // operand and the row-side factors. K-steps run outermost, so the
          // row side of a K-step is formed once for every pair of the run;
          // each tile still accumulates its K-steps in order.
          constexpr int MAXI = NW == 4 ? 3 : 2;      // longest run (gram_run)
          const float br = sBeta[r];
          f32x4 accL[MAXI], accB[MAXI];
#pragma unroll
          for (int t = 0; t < MAXI; ++t) { accL[t] = f32x4{0, 0, 0, 0}; accB[t] = f32x4{0, 0, 0, 0}; }
#pragma unroll
          for (int ks = 0; ks < D / 32; ++ks) {
            const int k0 = 32 * ks + 8 * g;
            float kraw[8], qraw[8] = {};
            if constexpr (BF16) {
              bf16x8_to_f32(raw_chunk<D>(regA + L::A_RK, r, 4 * ks + g, r < n), kraw);
              if constexpr (!MAP) bf16x8_to_f32(raw_chunk<D>(regA + L::A_RQ, r, 4 * ks + g, r < n), qraw);
            } else {
              const f16x8 kh16 = *reinterpret_cast<const f16x8*>(sRK + r * L::LDQ + k0);
#pragma unroll
              for (int e = 0; e < 8; ++e) kraw[e] = (float)kh16[e];
              if constexpr (!MAP) {
                const f16x8 qh16 = *reinterpret_cast<const f16x8*>(sRQ + r * L::LDQ + k0);
#pragma unroll
                for (int e = 0; e < 8; ++e) qraw[e] = (float)qh16[e];
              }
            }
            float kv[8], qv[8], gref[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int kk = k0 + e;
              gref[e] = sG[(16 * R) * L::LDG + kk];
              const float f = exp2_hw(sG[r * L::LDG + kk] - gref[e]);
              kv[e] = kraw[e] * f;
              qv[e] = qraw[e] * f;
            }
            bf16x8 kh, kl, qh, ql;
            split8_bf16(kv, kh, kl);
            if constexpr (!MAP) split8_bf16(qv, qh, ql);
#pragma unroll
            for (int t = 0; t < MAXI; ++t) {
              const int I = I0 + t;
              if (I > I1) break;                     // (uniform)
              const int i = 16 * I + l16;            // this lane's row of the column block
              float iraw[8];
              if constexpr (BF16) {
                bf16x8_to_f32(raw_chunk<D>(regA + L::A_RK, i, 4 * ks + g, i < n), iraw);
              } else {
                const f16x8 ih16 = *reinterpret_cast<const f16x8*>(sRK + i * L::LDQ + k0);
#pragma unroll
                for (int e = 0; e < 8; ++e) iraw[e] = (float)ih16[e];
              }
              float iv[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) iv[e] = iraw[e] * exp2_hw(gref[e] - sG[i * L::LDG + k0 + e]);
              bf16x8 ih, il;
              split8_bf16(iv, ih, il);
              if constexpr (!WU) {
                accL[t] = mfma_bf16(ih, kh, accL[t]);
                accL[t] = mfma_bf16(ih, kl, accL[t]);
                accL[t] = mfma_bf16(il, kh, accL[t]);
              }
              if constexpr (!MAP) {
                accB[t] = mfma_bf16(ih, qh, accB[t]);
                accB[t] = mfma_bf16(ih, ql, accB[t]);
                accB[t] = mfma_bf16(il, qh, accB[t]);
              }
            }
          }
#pragma unroll
          for (int t = 0; t < MAXI; ++t) {
            const int I = I0 + t;
            if (I > I1) break;                       // (uniform)
            const int i0 = 16 * I + 4 * g;
            f32x4 lv;
            f16x4 bv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              lv[e] = (i0 + e < r) ? accL[t][e] * br : 0.f;
              bv[e] = (_Float16)((i0 + e <= r) ? accB[t][e] : 0.f);
            }
            if constexpr (!WU) *reinterpret_cast<f32x4*>(sL + r * L::LDL + i0) = lv;
            if constexpr (!MAP) *reinterpret_cast<f16x4*>(sB + r * L::LDT + i0) = bv;
            if (!WU && I == R) {
              // diagonal tile: L_RR^T also into its upper triangle (column i
              // of L_RR becomes row i there); issued after the row stores, so
              // it lands after their zeros
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (i0 + e < r) sL[(i0 + e) * L::LDL + r] = lv[e];
            }
          }
        }
      }
      int d0, d1;
      if (!WU && gram_diag<NW, PER_KEY>(wave, d0, d1)) {
        // Replace L_bb by the inverse of the unit lower block I + L_bb for the
        // diagonal blocks this wavefront computed: lane groups 0-1 take block
        // d0, 2-3 block d1 (the same block when it inverts one: both halves
        // then store the same values), one column j per lane (groups 0 and 2
        // store). Right-looking: once x_i is final, every later row r takes
        // -L[r][i] x_i, read from row i of the transposed copy in the block's
        // upper triangle.
        __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): the tiles are in LDS
        __builtin_amdgcn_wave_barrier();
        const int b = g < 2 ? d0 : d1;
        float* Lb = sL + (16 * b) * L::LDL + 16 * b;
        float x[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) x[rr] = (rr == l16) ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < 15; ++i) {
          float col[16];                             // col[r] = L[r][i] for r > i
#pragma unroll
          for (int q4 = i / 4; q4 < 4; ++q4) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(Lb + i * L::LDL + 4 * q4);
            col[4 * q4] = t[0]; col[4 * q4 + 1] = t[1]; col[4 * q4 + 2] = t[2]; col[4 * q4 + 3] = t[3];
          }
#pragma unroll
          for (int rr = i + 1; rr < 16; ++rr) x[rr] -= col[rr] * x[i];
        }
        __builtin_amdgcn_wave_barrier();
        if ((g & 1) == 0) {
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) Lb[rr * L::LDL + l16] = x[rr];
        }
      }
    }
    if constexpr (WU) {
#pragma unroll
      for (int j = 0; j < W_PER_T; ++j) {
        const int e = tid + j * NT;
        if (e < W_VEC) reinterpret_cast<f32x4*>(sW)[e] = wreg[j];
      }
    }
    __syncthreads();

    if constexpr (!WU) {
      // ---- P4: A = (I + L)^-1, written as T~ = A Diag(beta) (fp16 hi + lo) --
      // The diagonal blocks A_RR are in place (P3). Block column I of the
      // off-diagonal part is one dependent chain on wavefront I (I = 0, 1, 2),
      //   A_RI = -A_RR (sum_{I<=m<R} L_Rm A_mI),   R = I+1 .. 3,
      // on fp32 MFMA with the column's blocks kept in accumulator registers;
      // each A_RI goes straight into T~.
      // The other wavefronts write the diagonal blocks of T~ and zero the
      // blocks above the diagonal. Meanwhile every wavefront stages V^T.
      {
        const int wv = __builtin_amdgcn_readfirstlane(wave);
        if (wv == 0) inverse_column<0, L>(sL, sBeta, sTh, sTl, lane);
        else if (wv == 1) inverse_column<1, L>(sL, sBeta, sTh, sTl, lane);
        else if (wv == 2) inverse_column<2, L>(sL, sBeta, sTh, sTl, lane);
        else inverse_rest<NW, L>(sL, sBeta, sTh, sTl, wv - 3, lane);
      }
      // V^T [v][c] into region A (G and raw q, k are dead after P3)
      {
#pragma unroll
        for (int j = 0; j < CR::GPT; ++j) {
          const int gi = tid + j * NT;
          const int c = gi / (D / 8), k8 = gi % (D / 8);
          float x[8];
          if constexpr (v_in_lds) {
            // staged bf16 rows [64][D] (unpadded); rows >= n are stale and zeroed here
            const uint4 vw = *reinterpret_cast<const uint4*>(smem + L::OFF_QT + (c * D + 8 * k8) * 2);
            const uint32_t vv4[4] = {vw.x, vw.y, vw.z, vw.w};
            const bool live = c < n;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x[2 * e] = live ? bf16_bits_to_f32(vv4[e] & 0xFFFFu) : 0.f;
              x[2 * e + 1] = live ? bf16_bits_to_f32(vv4[e] >> 16) : 0.f;
            }
          } else {
            unpack_group<BF16>(regs.v[j], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = c < n ? x[e] : 0.f;   // rows past n repeat row n - 1
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) sVT[(8 * k8 + e) * L::LDT + swz(8 * k8 + e, c)] = (_Float16)x[e];
        }
      }
      __syncthreads();
      load_chunk_rows<D, BF16, PER_KEY, NT>(regs, a, tok_next, n_next, h, tid, v_in_regs);

      // ---- P5: W = T~ (K * 2^G), U' = T~ V --------------------------------------
      // W[:, 16kt..16kt+15] for kt = wave, wave + NW, ... and U' = T~ V for the
      // wavefront's own value slices (K = 64), sharing each T~ hi/lo tile read;
      // U' stays in registers for P6. W is formed transposed (K^T as the A
      // operand), so a lane holds four consecutive columns of one row of W.
      {
        f32x4 acc[KT / NW][4];
#pragma unroll
        for (int kj = 0; kj < KT / NW; ++kj)
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) acc[kj][ct] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl)
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) Up[sl][ct] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          f16x8 th[4], tl[4], bk[KT / NW], bv[SPW];
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            th[ct] = ld_std(sTh, L::LDTT, 16 * ct, 32 * ks, lane);
            tl[ct] = ld_std(sTl, L::LDTT, 16 * ct, 32 * ks, lane);
          }
#pragma unroll
          for (int kj = 0; kj < KT / NW; ++kj) bk[kj] = ld_std_swz(sKhT, L::LDT, 16 * (wave + NW * kj), 32 * ks, lane);
#pragma unroll
          for (int sl = 0; sl < SPW; ++sl) bv[sl] = ld_std_swz(sVT, L::LDT, 16 * (SPW * wave + sl), 32 * ks, lane);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
            for (int kj = 0; kj < KT / NW; ++kj) {
              acc[kj][ct] = mfma_f16(bk[kj], th[ct], acc[kj][ct]);
              acc[kj][ct] = mfma_f16(bk[kj], tl[ct], acc[kj][ct]);
            }
#pragma unroll
            for (int sl = 0; sl < SPW; ++sl) {
              Up[sl][ct] = mfma_f16(th[ct], bv[sl], Up[sl][ct]);
              Up[sl][ct] = mfma_f16(tl[ct], bv[sl], Up[sl][ct]);
            }
          }
        }
        // lane (g, l16): W[16ct + l16][16kt + 4g .. +3], one 8-byte write per
        // tile; the map pass keeps this chunk's W (the LDS image) from here too
#pragma unroll
        for (int kj = 0; kj < KT / NW; ++kj)
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            const f16x4 w4 = {(_Float16)acc[kj][ct][0], (_Float16)acc[kj][ct][1], (_Float16)acc[kj][ct][2],
                              (_Float16)acc[kj][ct][3]};
            const int off = (16 * ct + l16) * L::LDQ + 16 * (wave + NW * kj) + 4 * g;
            *reinterpret_cast<f16x4*>(sW + off) = w4;
            if constexpr (MAP)
              *reinterpret_cast<f16x4*>(wu_base + (int64_t)ch * WU_BYTES + 2 * off) = w4;
          }
        if constexpr (MAP) {
          // and its U' (one accumulator tile per lane): issued before the
          // barrier, so the record drains while the other wavefronts finish P5
          f32x4* up = reinterpret_cast<f32x4*>(wu_base + (int64_t)ch * WU_BYTES + W_BYTES);
#pragma unroll
          for (int sl = 0; sl < SPW; ++sl)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) up[((SPW * wave + sl) * 4 + ct) * 64 + lane] = Up[sl][ct];
        }
      }
      __syncthreads();
    }  // !WU: P4, P5


    // WU: U' (fetched at the chunk start) has long arrived; waiting for it here
    // keeps the compiler from waiting for the prefetch below before P6 uses U'
    if constexpr (WU) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

    // prefetch the next chunk's raw inputs while the chain runs (bf16 q, k go
    // to the raw K/Q region, which P6 does not read)
    if constexpr (WU) load_chunk_rows<D, BF16, PER_KEY, NT>(regs, a, tok_next, n_next, h, tid, v_in_regs);
    if (ch + 1 < n_chunks) {
      if constexpr (BF16) {
        const int64_t row0 = ((tok0 + C) * a.H + h) * D;
        const int64_t rowq0 = ((tok0 + C) * Hq + hq) * D;
        if constexpr (v_in_lds)
          stage_rows_lds<D, NW>(static_cast<const uint16_t*>(a.v) + row0, HDu, n_next, smem + L::OFF_QT,
                            wave, lane);
        stage_rows_lds_swz<D, NW>(static_cast<const uint16_t*>(a.k) + rowq0, HDqu, n_next, regA + L::A_RK,
                                  wave, lane);
        if constexpr (!MAP)
          stage_rows_lds_swz<D, NW>(static_cast<const uint16_t*>(a.q) + rowq0, HDqu, n_next, regA + L::A_RQ,
                                    wave, lane);
      }
    }



    // ---- P6: state passing for this wavefront's slices ---------------------
    // Every A-operand tile read from LDS (T~, W, Q~, B, K~^T) feeds the MFMAs of
    // all SPW slices of the wavefront, which divides the LDS read traffic by SPW.
    // Operand tiles are read in batches ahead of their MFMAs (the scheduling
    // barriers keep each batch of reads in flight together).
    {
      // U starts as U' (from P5) for the first SPW slices, zero for M slices:
      // rows c (4 tiles), column v = 16 slice + l16
      f32x4 U[NSL][4];
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) U[sl][ct] = sl < SPW ? Up[sl % SPW][ct] : f32x4{0, 0, 0, 0};
      // S0^T as the permuted-K operand (fp16), shared by W S0^T and Q~ S0^T;
      // U = U' - W S0^T accumulates W (-S0^T) into U directly.
      f16x8 sop[NSL][D / 32];
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) sop[sl][ks] = pack_perm(ST[sl][2 * ks], ST[sl][2 * ks + 1]);
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        f16x8 w[4], nsop[NSL];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) w[ct] = ld_perm(sW, L::LDQ, 16 * ct, 32 * ks, lane);
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) nsop[sl] = -sop[sl][ks];
        if constexpr (!WU) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int sl = 0; sl < NSL; ++sl) U[sl][ct] = mfma_f16(w[ct], nsop[sl], U[sl][ct]);
      }
      // U as hi + lo permuted-K operands (K = chunk position, 2 steps)
      f16x8 uh[NSL][2], ul[NSL][2];
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) split_perm(U[sl][2 * ks], U[sl][2 * ks + 1], uh[sl][ks], ul[sl][ks]);
      if constexpr (out_mode) {
        // O^T = S0 Q~^T + U^T B^T, one 16-token tile at a time. MFMA's A and B
        // operands share one lane layout, so the S0^T and U operands above serve
        // as A and the Q~ and B tiles as B: lane (g, l16) then holds
        // O[token 16ct + l16][values 16 slice + 4g .. +3], one 16-byte store.
        const int64_t obase = tok0 * HD + (int64_t)h * D + 16 * SPW * wave + 4 * g;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          f16x8 qa[D / 32], ba[2];
#pragma unroll
          for (int ks = 0; ks < D / 32; ++ks) qa[ks] = ld_perm(sQt, L::LDQ, 16 * ct, 32 * ks, lane);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) ba[ks] = ld_perm(sB, L::LDT, 16 * ct, 32 * ks, lane);
          if constexpr (!WU) __builtin_amdgcn_sched_barrier(0);
          f32x4 OT[SPW];
#pragma unroll
          for (int sl = 0; sl < SPW; ++sl) OT[sl] = f32x4{0, 0, 0, 0};
#pragma unroll
          for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
            for (int sl = 0; sl < SPW; ++sl) OT[sl] = mfma_f16(sop[sl][ks], qa[ks], OT[sl]);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int sl = 0; sl < SPW; ++sl) {
              OT[sl] = mfma_f16(uh[sl][ks], ba[ks], OT[sl]);
              OT[sl] = mfma_f16(ul[sl][ks], ba[ks], OT[sl]);
            }
          const int c = 16 * ct + l16;                 // this lane's token in the chunk
          if constexpr (EPI == EPI_O) {
            if (c < n) {
              float* orow = a.o + obase + (int64_t)c * HD;
#pragma unroll
              for (int sl = 0; sl < SPW; ++sl) *reinterpret_cast<f32x4*>(orow + 16 * sl) = OT[sl];
            }
          } else {
            // this wavefront's share of row c's sum of squares, formed as the
            // back end's lanes of 8 values form theirs: lane group g holds
            // values 4g .. 4g+3 of the slice, so an odd group continues its
            // even neighbour's running sum (v_permlane16_swap: odd rows of
            // the first operand come from even rows of the second), and groups
            // g and g ^ 2 then add (v_permlane32_swap exchanges the halves)
            static_assert(SPW == 1, "one slice a wavefront");
            float s0 = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) s0 = __builtin_fmaf(OT[0][e], OT[0][e], s0);
            float s1 = __uint_as_float(
                __builtin_amdgcn_permlane16_swap(__float_as_uint(s0), __float_as_uint(s0), false, false)[0]);
#pragma unroll
            for (int e = 0; e < 4; ++e) s1 = __builtin_fmaf(OT[0][e], OT[0][e], s1);
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(s1), __float_as_uint(s1), false, false);
            sEP[(g & 1) ? NW * c + wave : NW * C + lane] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            Oh[ct] = OT[0];
          }
        }
      }
      // S^T <- 2^(G_n) S^T + K~^T U, four row tiles per batch
#pragma unroll
      for (int kb = 0; kb < KT; kb += 4) {
        f16x8 ka[4][2];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) ka[t][ks] = ld_perm_swz(sKtT, L::LDT, 16 * (kb + t), 32 * ks, lane);
        if constexpr (!WU) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const f32x4 gam = *reinterpret_cast<const f32x4*>(sGam + 16 * (kb + t) + 4 * g);
#pragma unroll
          for (int sl = 0; sl < NSL; ++sl) ST[sl][kb + t] *= gam;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int sl = 0; sl < NSL; ++sl) {
              ST[sl][kb + t] = mfma_f16(ka[t][ks], uh[sl][ks], ST[sl][kb + t]);
              ST[sl][kb + t] = mfma_f16(ka[t][ks], ul[sl][ks], ST[sl][kb + t]);
            }
        }
      }
    }

    // snapshot after this chunk if the sequence position is a multiple of the interval
    if (out_mode && a.interval > 0) {   // OUT only (constant false in MAP)
      const int64_t pos = item.tok_in_seq + (int64_t)ch * C + n;   // tokens of the sequence done
      if (pos % a.interval == 0) {
        const int64_t slot = item.snap_base + pos / a.interval - 1;
        float* dst = a.snapshots + (slot * a.H + h) * DD;
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl)
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
            *reinterpret_cast<f32x4*>(dst + (16 * (SPW * wave + sl) + l16) * D + 16 * kt + 4 * g) = ST[sl][kt];
      }
    }
    if constexpr (PER_KEY) local_scan(n_next);     // the next chunk's (P1 of this one read sPart)
    if constexpr (BF16) __builtin_amdgcn_s_waitcnt(0);   // staged rows have landed in LDS
    __syncthreads();
  }

  if constexpr (EPI != EPI_O) {
    // the back end of the last chunk (its shares are in LDS since the loop's
    // last barrier)
    if (n_chunks > 0) {
      const int lane = tid % 64, g = lane >> 4, l16 = lane & 15;
      const int64_t tl = item.tok_begin + (int64_t)(n_chunks - 1) * C;
      const int nl = item.n_tokens - (n_chunks - 1) * C;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) epi_tile(ct, tl * HD + (int64_t)h * D + 16 * wave + 4 * g, nl, g, l16);
    }
  }
  // end of the item: the final state (OUT, last segment of the sequence) or the
  // segment's map (MAP: N rows from the first SPW slices, M rows from the rest)
  if constexpr (!MAP) {
    if (item.seg == item.n_segs - 1) {
      float* dst = a.final_state + ((int64_t)item.seq * a.H + h) * DD;
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
          *reinterpret_cast<f32x4*>(dst + (16 * (SPW * wave + sl) + l16) * D + 16 * kt + 4 * g) = ST[sl][kt];
    }
  } else {
    float* maps = a.seg_maps + ((int64_t)item_idx * a.H + h) * 2 * DD;   // [M, N]
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      float* dst = maps + (sl < SPW ? DD : 0);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
        *reinterpret_cast<f32x4*>(dst + (16 * (SPW * wave + sl % SPW) + l16) * D + 16 * kt + 4 * g) =
            ST[sl][kt];
    }
  }
}

// ---- Pass 1 (segment maps), scalar gate, bf16 inputs, d = 128 -------------
// Every product that contracts over the 64 chunk rows (W = T~ (K * 2^G),
// U' = T~ V and the state update with K~^T) takes its K or V operand straight
// from the raw token-major rows staged in LDS, through the LDS transpose read
// (ds_read_b64_tr_b16: in each group of 16 lanes, lane j names the 8 bytes at
// row base + j/4, columns c0 + 4 (j % 4) .. +3, and lane i receives column
// c0 + i of those four rows, one row per element). No transposed copy of K or
// V is written. The scalar gate's decay factors go where the operands are
// formed instead: 2^G_c multiplies the K operand of W in registers, and
// 2^(G_n - G_c) multiplies row c of U before the state update,
//     (K * 2^(G_n - G))^T U = K^T (2^(G_n - G) * U),
// whose K^T operand is then the raw bf16 row data itself (U as bf16 hi + lo).

// Eight raw values x[c][col0 + (lane % 16)] of staged rows [64][D] bf16
// (chunk-permuted, raw_swz): c = r0 + {0..3} from the first transpose read,
// r1 + {0..3} from the second; r0 and r1 are this lane group's row bases.
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef int i32x4 __attribute__((ext_vector_type(4)));
template <int D>
__device__ __forceinline__ bf16x8 tr_rows(const unsigned char* raw, int r0, int r1, int col0, int lane) {
  const int j = lane & 15;
  const int col = col0 + 4 * (j & 3);
  auto piece = [&](int r) __attribute__((always_inline)) {
    const int rr = r + (j >> 2);
    const unsigned char* p = raw + rr * (D * 2) + (((col >> 3) ^ raw_swz<D>(rr)) << 4) + ((col >> 2) & 1) * 8;
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
  };
  const bf16x4_t a = piece(r0), b = piece(r1);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ f16x8 bf16x8_to_f16(bf16x8 x, const float (&scale)[8]) {
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (_Float16)((float)x[e] * scale[e]);
  return r;
}

// Twelve wavefronts in two roles. Wavefronts 4-11 (producers) run the phases
// that do not depend on the state, for chunk c+1, on the eight-wavefront
// schedules: the Gram tiles and diagonal inversions, the inverse T~, and W and
// U' (into LDS for the chain and into the stored record). The producers also
// carry the M rows (16 each). M enters U only through its fp16 image; once
// that image is zero in every lane of a wavefront (every |M| entry at most
// 2^-25), its U is zero and its step is exactly M <- 2^G_n M, and since
// 2^G_n <= 1 the image stays zero, so the wavefront stops forming products
// for it. Wavefronts 0-3 (chain) run the N rows (32 each) through chunk c
// meanwhile. A chunk takes three barrier intervals:
//   A: chain: U = U' - W S0^T and the state update (chunk c)
//      producers: the fetch of c+1's v rows and c+2's k rows into registers,
//      the Gram tiles of c+1 and their inversions
//   B: producers: c+1's v rows into LDS, the inverse T~ of c+1; the M step
//      (chunk c)
//   C: producers: W and U' of c+1, c+2's k rows into LDS; chain wavefront 0:
//      the decay scan of c+2 (the chain is otherwise idle in B and C)
// The raw k rows are double-buffered: chunk c+2's wait in registers until
// interval C, when the chain and the M step are done with chunk c's buffer.
// The small arrays are triple-buffered, W double-buffered. The raw rows travel
// through registers, not LDS-bound loads: a barrier after an LDS-bound load
// waits for it to land. Each product accumulates its K-steps in a fixed
// order, so the record and the maps do not depend on the timing of the roles.
template <int D>
struct LdsMapChain {
  using L = Lds<D>;
  static constexpr int RK = 0;                                  // raw k [2][64][D] bf16 (raw_swz)
  static constexpr int RV = RK + 2 * C * D * 2;                 // raw v [64][D] bf16 (raw_swz)
  static constexpr int LM = RV + C * D * 2;                     // L / A [64][LDL] f32
  static constexpr int TH = LM + C * L::LDL * 4;                // T~ hi [64][LDTT] f16
  static constexpr int TL = TH + C * L::LDTT * 2;               // T~ lo
  static constexpr int WB = TL + C * L::LDTT * 2;               // W [2][64][LDQ] f16 (the stored image)
  static constexpr int UP = WB + 2 * C * L::LDQ * 2;            // U' [slice 8][tile 4][lane 64] f32x4
  static constexpr int SM = UP + (D / 16) * 4 * 64 * 16;        // [3] x {G, 2^G, 2^(G_n-G), beta}[64], 2^G_n
  static constexpr int SMF = 4 * C + 4;                         // floats per small-array buffer
  static constexpr int TOTAL = SM + 3 * SMF * 4;
  static_assert(RV % 512 == 0 && LM % 512 == 0 && TH % 512 == 0 && TL % 512 == 0 && WB % 512 == 0 &&
                UP % 512 == 0 && (C * L::LDQ * 2) % 512 == 0, "buffers start on a 512-byte boundary (bank alignment)");
};

template <int D>
__global__ __launch_bounds__(768) __attribute__((amdgpu_waves_per_eu(3, 3)))
void prefill_map_chain_kernel(PrefillArgs a) {
  static_assert(D == 128, "four chain wavefronts of 32 N rows, eight producers of 16 M rows");
  constexpr int NC = 4, NP = 8;                  // chain and producer wavefronts
  constexpr int KT = D / 16;
  constexpr int LPR = D / 8;                     // lanes per raw row (16 bytes each)
  constexpr int RPI = 64 / LPR;                  // raw rows per wavefront instruction
  constexpr int RI = C / RPI / NP;               // raw-row instructions per producer and tensor
  static_assert(RI * RPI * NP == C, "every producer moves the same number of rows");
  using L = Lds<D>;
  using P = LdsMapChain<D>;
  extern __shared__ __align__(16) unsigned char smem[];
  float* sL = reinterpret_cast<float*>(smem + P::LM);
  _Float16* sTh = reinterpret_cast<_Float16*>(smem + P::TH);
  _Float16* sTl = reinterpret_cast<_Float16*>(smem + P::TL);
  unsigned char* rawV = smem + P::RV;
  f32x4* sUp = reinterpret_cast<f32x4*>(smem + P::UP);
  auto rawK = [&](int ch) { return smem + P::RK + (ch & 1) * C * D * 2; };
  auto sWb = [&](int ch) { return reinterpret_cast<_Float16*>(smem + P::WB + (ch & 1) * C * L::LDQ * 2); };
  auto sSm = [&](int ch) { return reinterpret_cast<float*>(smem + P::SM) + (ch % 3) * P::SMF; };

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const bool chain = wave < NC;                  // (uniform per wavefront)
  const int pw = wave - NC;                      // producer index
  int tid = threadIdx.x, lane = tid % 64, g = lane >> 4, l16 = lane & 15;
  auto refresh = [&]() __attribute__((always_inline)) {
    asm volatile("" : "+v"(tid));
    lane = tid % 64;
    g = lane >> 4;
    l16 = lane & 15;
  };
  const int item_idx = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const PrefillItem item = work_item(a, item_idx);
  if (item.n_segs <= 1) return;                  // (uniform) whole sequences need no map
  constexpr int W_BYTES = (int)wu_w_bytes(D);
  static_assert(W_BYTES == C * L::LDQ * 2, "stored W layout");
  constexpr int64_t WU_BYTES = (int64_t)wu_chunk_bytes(D);
  unsigned char* wu_base =
      static_cast<unsigned char*>(a.seg_wu) + ((int64_t)item_idx * a.H + h) * a.seg_chunks * WU_BYTES;
  const int64_t DD = (int64_t)D * D;
  const uint32_t HDu = (uint32_t)a.H * D;
  const int n_chunks = (item.n_tokens + C - 1) / C;
  if (n_chunks == 0) return;                     // (uniform; a segment is never empty)
  auto chunk_len = [&](int ch) { return min(C, item.n_tokens - ch * C); };

  // ---- producer phases ----------------------------------------------------------
  i32x4 carry_k[RI], carry_v[RI];
  // raw rows of chunk ch into registers, in the order stage_rows_lds_swz lays
  // them out (instruction i = pw + NP j: rows i RPI + lane / LPR; lane l holds
  // the 16 bytes that land at 1024 i + 16 l); rows past the end are row 0
  auto fetch_rows = [&](const void* src, int ch, i32x4 (&carry)[RI]) __attribute__((always_inline)) {
    const int n = chunk_len(ch);
    const uint16_t* base = static_cast<const uint16_t*>(src) + ((item.tok_begin + (int64_t)ch * C) * a.H + h) * D;
#pragma unroll
    for (int j = 0; j < RI; ++j) {
      const int i = pw + NP * j;
      const int row = i * RPI + lane / LPR;
      const uint32_t off = (uint32_t)(row < n ? row : 0) * HDu + 8u * (uint32_t)((lane % LPR) ^ raw_swz<D>(row));
      carry[j] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(base + off));
    }
  };
  auto put_rows = [&](unsigned char* dst, const i32x4 (&carry)[RI]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < RI; ++j) *reinterpret_cast<i32x4*>(dst + 1024 * (pw + NP * j) + 16 * lane) = carry[j];
  };
  // alpha and beta of token `lane` of a later chunk (every wavefront of the
  // role that scans them loads them)
  float pre_alpha = 1.f, pre_beta = 0.f;
  auto fetch_ab = [&](int ch) __attribute__((always_inline)) {
    const int64_t t = (item.tok_begin + (int64_t)ch * C + min(lane, chunk_len(ch) - 1)) * a.H + h;
    pre_alpha = a.alpha[t];
    pre_beta = a.beta[t];
  };
  // the loaded alpha and beta are waited for here (p1 can then follow record
  // stores without waiting for them)
  auto land_ab = [&]() __attribute__((always_inline)) { asm volatile("" : "+v"(pre_alpha), "+v"(pre_beta)); };
  // P1: cumulative log2 decay of chunk ch (by the wavefront with `mine` set:
  // producer 0 in the prologue, chain wavefront 0 in the loop)
  auto p1 = [&](int ch, bool mine) __attribute__((always_inline)) {
    if (mine) {
      const int n = chunk_len(ch);
      float* sm = sSm(ch);
      const float gcum = wave_inclusive_scan(log2_hw(lane < n ? pre_alpha : 1.f), lane);
      const float gl = __shfl(gcum, C - 1);
      sm[lane] = gcum;                                   // G
      sm[C + lane] = lane < n ? exp2_hw(gcum) : 0.f;      // 2^G (0 past the chunk end)
      sm[2 * C + lane] = exp2_hw(gl - gcum);              // 2^(G_n - G)
      sm[3 * C + lane] = lane < n ? pre_beta : 0.f;       // beta
      if (lane == 0) sm[4 * C] = exp2_hw(gl);             // 2^G_n
    }
  };
  // P3: Gram tiles L = beta_r K K^T 2^(G_r - G_i) (strictly lower) on the
  // eight-wavefront run schedule, then the inverses of the diagonal blocks
  auto p3 = [&](int ch) __attribute__((always_inline)) {
    const int n = chunk_len(ch);
    const unsigned char* rk = rawK(ch);
    const float* sGs = sSm(ch);
    const float* sBeta = sGs + 3 * C;
#pragma unroll
    for (int run = 0; run < 2; ++run) {
      int R, I0, I1;
      if (!gram_run<NP, false>(pw, run, R, I0, I1)) break;
      const int r = 16 * R + l16;
      bf16x8 kr[D / 32];
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) kr[ks] = as_bf16x8(raw_chunk<D>(rk, r, 4 * ks + g, r < n));
      const float gr = sGs[r], br = sBeta[r];
      for (int I = I0; I <= I1; ++I) {
        f32x4 accL = {0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          const int i = 16 * I + l16;
          accL = mfma_bf16(as_bf16x8(raw_chunk<D>(rk, i, 4 * ks + g, i < n)), kr[ks], accL);
        }
        const int i0 = 16 * I + 4 * g;
        const f32x4 gi = *reinterpret_cast<const f32x4*>(sGs + i0);
        f32x4 lv;
#pragma unroll
        for (int e = 0; e < 4; ++e) lv[e] = (i0 + e < r) ? accL[e] * exp2_hw(fminf(gr - gi[e], 0.f)) * br : 0.f;
        *reinterpret_cast<f32x4*>(sL + r * L::LDL + i0) = lv;
        if (I == R) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (i0 + e < r) sL[(i0 + e) * L::LDL + r] = lv[e];
        }
      }
    }
    int d0, d1;
    if (gram_diag<NP, false>(pw, d0, d1)) {
      __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0): the tiles are in LDS
      __builtin_amdgcn_wave_barrier();
      const int b = g < 2 ? d0 : d1;
      float* Lb = sL + (16 * b) * L::LDL + 16 * b;
      float x[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) x[rr] = (rr == l16) ? 1.f : 0.f;
      // row i of the transposed copy is read one step ahead of its use; its
      // offset is tied to x[i-1] through an empty asm, so the reads cannot be
      // hoisted together (the whole block in registers spills at three
      // wavefronts per SIMD)
      f32x4 rows[2][4];
      auto fetch = [&](int i) __attribute__((always_inline)) {
        int off = i * L::LDL;
        if (i > 0) asm volatile("" : "+v"(off) : "v"(x[i - 1]));
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          if (q4 >= i / 4) rows[i & 1][q4] = *reinterpret_cast<const f32x4*>(Lb + off + 4 * q4);
      };
      fetch(0);
#pragma unroll
      for (int i = 0; i < 15; ++i) {
        if (i + 1 < 15) fetch(i + 1);
#pragma unroll
        for (int rr = i + 1; rr < 16; ++rr) x[rr] -= rows[i & 1][rr / 4][rr % 4] * x[i];
      }
      __builtin_amdgcn_wave_barrier();
      if ((g & 1) == 0) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) Lb[rr * L::LDL + l16] = x[rr];
      }
    }
  };
  // P4: T~ = (I + L)^-1 Diag(beta): column chains on producers 0-2, the
  // diagonal blocks and zeros on producers 3-7
  auto p4 = [&](int ch) __attribute__((always_inline)) {
    const float* sBeta = sSm(ch) + 3 * C;
    if (pw == 0) inverse_column<0, L>(sL, sBeta, sTh, sTl, lane);
    else if (pw == 1) inverse_column<1, L>(sL, sBeta, sTh, sTl, lane);
    else if (pw == 2) inverse_column<2, L>(sL, sBeta, sTh, sTl, lane);
    else inverse_rest<NP, L>(sL, sBeta, sTh, sTl, pw - 3, lane);
  };
  // P5: W^T tile kt = pw and U' for value slice pw of chunk ch: W into LDS and
  // the record, U' into LDS (for the chain) and the record
  auto p5 = [&](int ch) __attribute__((always_inline)) {
    const unsigned char* rk = rawK(ch);
    const float* sDec = sSm(ch) + C;
    _Float16* sW = sWb(ch);
    f32x4 accW[4], Up[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) { accW[ct] = f32x4{0, 0, 0, 0}; Up[ct] = f32x4{0, 0, 0, 0}; }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      f16x8 th[4], tl[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        th[ct] = ld_std(sTh, L::LDTT, 16 * ct, 32 * ks, lane);
        tl[ct] = ld_std(sTl, L::LDTT, 16 * ct, 32 * ks, lane);
      }
      const int c0 = 32 * ks + 8 * g;
      float dec[8];
      {
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(sDec + c0);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(sDec + c0 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) { dec[e] = d0[e]; dec[4 + e] = d1[e]; }
      }
      const float one[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
      const f16x8 bk = bf16x8_to_f16(tr_rows<D>(rk, c0, c0 + 4, 16 * pw, lane), dec);
      const f16x8 bv = bf16x8_to_f16(tr_rows<D>(rawV, c0, c0 + 4, 16 * pw, lane), one);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        accW[ct] = mfma_f16(bk, th[ct], accW[ct]);
        accW[ct] = mfma_f16(bk, tl[ct], accW[ct]);
        Up[ct] = mfma_f16(th[ct], bv, Up[ct]);
        Up[ct] = mfma_f16(tl[ct], bv, Up[ct]);
      }
    }
    unsigned char* rec = wu_base + (int64_t)ch * WU_BYTES;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const f16x4 w4 = {(_Float16)accW[ct][0], (_Float16)accW[ct][1], (_Float16)accW[ct][2], (_Float16)accW[ct][3]};
      const int off = (16 * ct + l16) * L::LDQ + 16 * pw + 4 * g;
      *reinterpret_cast<f16x4*>(sW + off) = w4;
      *reinterpret_cast<f16x4*>(rec + 2 * off) = w4;
    }
    f32x4* up = reinterpret_cast<f32x4*>(rec + W_BYTES);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      sUp[(pw * 4 + ct) * 64 + lane] = Up[ct];
      up[(pw * 4 + ct) * 64 + lane] = Up[ct];
    }
  };

  // ---- state steps (NS slices: two on the chain, one on a producer) -----------
  // U = U' - W S0^T of chunk ch (U' from LDS on the chain, zero for M), times
  // 2^(G_n - G_c) by row, as bf16 hi + lo permuted-K operands; false (nothing
  // formed) for an M slice whose fp16 image is zero
  bf16x8 uh[2][2], ul[2][2];
  auto ustep = [&](int ch, auto& ST) __attribute__((always_inline)) -> bool {
    constexpr int NS = sizeof(ST) / sizeof(ST[0]);
    const _Float16* sW = sWb(ch);
    const float* sRem = sSm(ch) + 2 * C;
    f16x8 sop[NS][D / 32];
#pragma unroll
    for (int sl = 0; sl < NS; ++sl)
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) sop[sl][ks] = pack_perm(ST[sl][2 * ks], ST[sl][2 * ks + 1]);
    if constexpr (NS == 1) {
      uint32_t bits = 0;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const i32x4 w4 = __builtin_bit_cast(i32x4, sop[0][ks]);
        bits |= (uint32_t)(w4[0] | w4[1] | w4[2] | w4[3]);
      }
      if (__builtin_amdgcn_ballot_w64((bits & 0x7FFF7FFFu) != 0) == 0) return false;   // +0 and -0
    }
    f32x4 U[NS][4];
#pragma unroll
    for (int sl = 0; sl < NS; ++sl)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        U[sl][ct] = NS == 1 ? f32x4{0, 0, 0, 0} : sUp[((2 * wave + sl) * 4 + ct) * 64 + lane];
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      f16x8 w[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) w[ct] = ld_perm(sW, L::LDQ, 16 * ct, 32 * ks, lane);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) U[sl][ct] = mfma_f16(w[ct], -sop[sl][ks], U[sl][ct]);
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const f32x4 rem = *reinterpret_cast<const f32x4*>(sRem + 16 * ct + 4 * g);
#pragma unroll
      for (int sl = 0; sl < NS; ++sl) U[sl][ct] *= rem;
    }
#pragma unroll
    for (int sl = 0; sl < NS; ++sl)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) split_tiles_bf16(U[sl][2 * ks], U[sl][2 * ks + 1], uh[sl][ks], ul[sl][ks]);
    return true;
  };
  // S^T <- 2^G_n S^T + K^T (2^(G_n - G) * U) of chunk ch (live: U was formed)
  auto update = [&](int ch, bool live, auto& ST) __attribute__((always_inline)) {
    constexpr int NS = sizeof(ST) / sizeof(ST[0]);
    const unsigned char* rk = rawK(ch);
    const float gam = sSm(ch)[4 * C];
#pragma unroll
    for (int kb = 0; kb < KT; kb += 4) {
      bf16x8 ka[4][2];
      if (live) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            ka[t][ks] = tr_rows<D>(rk, 32 * ks + 4 * g, 32 * ks + 16 + 4 * g, 16 * (kb + t), lane);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) ST[sl][kb + t] *= gam;
        if (live) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int sl = 0; sl < NS; ++sl) {
              ST[sl][kb + t] = mfma_bf16(ka[t][ks], uh[sl][ks], ST[sl][kb + t]);
              ST[sl][kb + t] = mfma_bf16(ka[t][ks], ul[sl][ks], ST[sl][kb + t]);
            }
        }
      }
    }
  };
  // The two roles run separate loops (each holds only its own state in
  // registers); both pass the same barriers: four in the prologue, three a
  // chunk.
  float* maps = a.seg_maps + ((int64_t)item_idx * a.H + h) * 2 * DD;   // [M, N]
  if (chain) {
    // N rows 32 wave + 16 sl + l16 from S = 0; S^T in accumulator layout
    f32x4 SN[2][KT];
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) SN[sl][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < 4; ++b) __syncthreads();                // the producers' prologue
    for (int ch = 0; ch < n_chunks; ++ch) {
      refresh();
      ustep(ch, SN);                             // interval A
      update(ch, true, SN);
      fetch_ab(min(ch + 2, n_chunks - 1));       // for the decay scan of chunk ch+2
      __syncthreads();
      __syncthreads();                           // interval B
      land_ab();                                 // interval C: the decay scan of ch+2
      if (ch + 2 < n_chunks) p1(ch + 2, wave == 0);   // (small arrays of chunk ch-1)
      __syncthreads();
    }
    refresh();
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
        *reinterpret_cast<f32x4*>(maps + DD + (32 * wave + 16 * sl + l16) * D + 16 * kt + 4 * g) = SN[sl][kt];
    return;
  }
  // producers: M rows 16 pw + l16 from the identity
  f32x4 SMr[1][KT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) SMr[0][kt][i] = (16 * pw + l16 == 16 * kt + 4 * g + i) ? 1.f : 0.f;

  // ---- prologue: chunk 0 prepared, chunk 1's k rows and decay scan -------------
  // Every fetch and every put of raw rows is unconditional (past the last
  // chunk they repeat it): the wait for a load then has the same count on
  // every path, where a load or a store under a branch makes the compiler
  // wait for all memory traffic in flight.
  const int last = n_chunks - 1;
  fetch_rows(a.k, 0, carry_k);
  fetch_rows(a.v, 0, carry_v);
  fetch_ab(0);
  put_rows(rawK(0), carry_k);
  put_rows(rawV, carry_v);
  p1(0, pw == 0);
  fetch_rows(a.k, min(1, last), carry_k);
  fetch_ab(min(1, last));
  __syncthreads();
  refresh();
  p3(0);
  put_rows(rawK(1), carry_k);
  land_ab();
  __syncthreads();
  refresh();
  p4(0);
  __syncthreads();
  refresh();
  p5(0);
  if (n_chunks > 1) p1(1, pw == 0);
  __syncthreads();

  bool m_live = true;                            // this wavefront's M image is nonzero
  for (int ch = 0; ch < n_chunks; ++ch) {
    const bool has_next = ch + 1 < n_chunks;
    refresh();
    // ---- interval A ---------------------------------------------------------
    fetch_rows(a.v, min(ch + 1, last), carry_v);
    if (has_next) p3(ch + 1);
    fetch_rows(a.k, min(ch + 2, last), carry_k); // (after P3: not live across it)
    __syncthreads();
    refresh();
    // ---- interval B ---------------------------------------------------------
    put_rows(rawV, carry_v);                     // v rows of chunk ch were read in the last interval C
    if (has_next) p4(ch + 1);
    if (m_live) m_live = ustep(ch, SMr);
    update(ch, m_live, SMr);
    __syncthreads();
    refresh();
    // ---- interval C ---------------------------------------------------------
    put_rows(rawK(ch + 2), carry_k);             // k rows of chunk ch were read in intervals A and B
    if (has_next) p5(ch + 1);
    __syncthreads();
  }
  refresh();
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
    *reinterpret_cast<f32x4*>(maps + (16 * pw + l16) * D + 16 * kt + 4 * g) = SMr[0][kt];
}

// ---- Pass 3, scalar gate, bf16 inputs, d = 128: chain and producer wavefronts
// Only P6 depends on the state; P1-P3 of a chunk (decay scan, Q~ and K~^T, the
// output Gram B) need its raw rows alone. In this form of pass 3 wavefronts
// 0-3 (one per SIMD) run the chain, each on 32 state rows (two slices), and
// wavefronts 4-7 prepare the next chunk: they fetch its raw q/k rows, alpha and
// stored W, scan its decay and form Q~, K~^T and B in the other half of a
// double buffer. A chain wavefront reads every shared operand once for both of
// its slices, so P6 reads half the LDS bytes of the eight-slice form. Each
// chunk takes two barrier intervals:
//   A: chain: U = U' - W S0^T (chunk c)
//      producers: raw rows of c+1 into LDS, its decay scan, the fetch of its W
//   B: chain: the fetch of U' (c+1), O and the state update (chunk c)
//      producers: Q~ and K~^T of c+1, the fetch of c+2's raw rows, B of c+1,
//      W of c+1 into LDS (the chain read chunk c's in interval A)
// The producers' fetch of raw rows sits after Q~ and K~^T: issued at the start
// of interval B it delays the chain's o stores, which share the compute
// unit's vector memory path with it (pass 3 then takes about 10 % longer).
// Everything this kernel moves through HBM is touched once (raw rows, stored
// W and U', o), so those accesses are nontemporal.
// Every product is the one the other pass-3 form computes, in the same order,
// so both give the same bits.
template <int D>
struct LdsPipe {
  using L = Lds<D>;
  static constexpr int QT = 0;                                  // Q~    [64][LDQ] f16
  static constexpr int KTT = QT + C * L::LDQ * 2;               // K~^T  [D][LDT] f16 (swizzled)
  static constexpr int BG = KTT + D * L::LDT * 2;               // B     [64][LDT] f16
  static constexpr int GS = BG + C * L::LDT * 2;                // G[64], 2^G[64], 2^(G_n-G)[64], 2^G_n[D] f32
  static constexpr int BUF = GS + ((3 * C + D) * 4 + 511) / 512 * 512;   // one buffer
  static constexpr int OFF_W = 2 * BUF;                         // W     [64][LDQ] f16 (the stored image)
  static constexpr int OFF_RK = OFF_W + C * L::LDQ * 2;         // raw k [64][D] bf16 (raw_swz)
  static constexpr int OFF_RQ = OFF_RK + C * D * 2;             // raw q
  static constexpr int TOTAL = OFF_RQ + C * D * 2;
  static_assert(BUF % 512 == 0 && OFF_W % 512 == 0, "buffers keep the bank alignment of the other form");
  // fused back end only: each chain wavefront's share of a row's sum of
  // squares [64][4] f32 (then 64 floats the lanes without a share write),
  // norm_w [D], and one chunk's output-gate logits [64][D] bf16, which the
  // chain overwrites in place with the bf16 output rows
  static constexpr int OFF_PART = TOTAL;
  static constexpr int OFF_NW = OFF_PART + (4 * C + 64) * 4;
  static constexpr int LDG = 2 * D + 16;                         // gate / output row stride (bytes)
  static constexpr int OFF_G = OFF_NW + D * 4;
  static constexpr int TOTAL_EPI = OFF_G + C * LDG;
};

template <int D, int EPI>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_wu_pipe_kernel(PrefillArgs a) {
  static_assert(D == 128, "four chain wavefronts of 32 state rows");
  constexpr int NC = 4, NP = 4;                  // chain and producer wavefronts
  constexpr int NPT = 64 * NP;                   // producer threads
  using L = Lds<D>;
  using P = LdsPipe<D>;
  constexpr int SPW = D / (16 * NC);             // state slices per chain wavefront
  constexpr int KT = D / 16;
  constexpr int LPR = D / 8;                     // lanes per raw row (16 bytes each)
  constexpr int RPI = 64 / LPR;                  // raw rows per wavefront instruction
  constexpr int RI = C / RPI / NP;               // raw-row instructions per producer and tensor
  static_assert(RI * RPI * NP == C, "every producer stages the same number of rows");
  constexpr int GPT = C * D / 8 / NPT;           // P2: 8-element groups per producer thread
  static_assert(GPT * 8 * NPT == C * D, "P2 covers the chunk");
  extern __shared__ __align__(16) unsigned char smem[];
  _Float16* sW = reinterpret_cast<_Float16*>(smem + P::OFF_W);
  unsigned char* rawK = smem + P::OFF_RK;
  unsigned char* rawQ = smem + P::OFF_RQ;
  [[maybe_unused]] float* sPart = reinterpret_cast<float*>(smem + P::OFF_PART);
  [[maybe_unused]] float* sNw = reinterpret_cast<float*>(smem + P::OFF_NW);
  [[maybe_unused]] unsigned char* sG = smem + P::OFF_G;

  const int wave = threadIdx.x / 64;
  const bool chain = wave < NC;                  // (uniform per wavefront)
  const int pw = wave - NC;                      // producer wavefront index
  // Per-lane indices (ptid: producer thread index) are refreshed from an
  // opaque copy of the thread index at every chunk: hoisted out of the loop,
  // the addresses derived from them would hold registers for the whole item.
  int tid = threadIdx.x, lane = tid % 64, g = lane >> 4, l16 = lane & 15, ptid = tid - 64 * NC;
  auto refresh = [&]() __attribute__((always_inline)) {
    asm volatile("" : "+v"(tid));
    lane = tid % 64;
    g = lane >> 4;
    l16 = lane & 15;
    ptid = tid - 64 * NC;
  };
  const int item_idx = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const PrefillItem item = work_item(a, item_idx);
  if (item.n_segs <= 1) return;                  // (uniform) whole sequences run in the other pass
  constexpr int W_BYTES = (int)wu_w_bytes(D);
  static_assert(W_BYTES == C * L::LDQ * 2, "stored W layout");
  constexpr int64_t WU_BYTES = (int64_t)wu_chunk_bytes(D);
  const unsigned char* wu_base =
      static_cast<const unsigned char*>(a.seg_wu) + ((int64_t)item_idx * a.H + h) * a.seg_chunks * WU_BYTES;
  const int64_t HD = (int64_t)a.H * D;
  const int64_t DD = (int64_t)D * D;
  const uint32_t HDu = (uint32_t)a.H * D;
  const int n_chunks = (item.n_tokens + C - 1) / C;
  if (n_chunks == 0) return;                     // (uniform; a segment is never empty)
  auto chunk_len = [&](int ch) { return min(C, item.n_tokens - ch * C); };

  // chain: start state of the segment (from the scan), S0^T in accumulator
  // layout; slice sl covers state rows 16 (SPW wave + sl) .. +15
  f32x4 ST[SPW][KT];
  if (chain) {
    const float* src = a.seg_states + ((int64_t)item_idx * a.H + h) * DD;
#pragma unroll
    for (int sl = 0; sl < SPW; ++sl) {
      const int row = 16 * (SPW * wave + sl) + l16;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) ST[sl][kt] = *reinterpret_cast<const f32x4*>(src + row * D + 16 * kt + 4 * g);
    }
  }
  // vmcnt(0): the start state has landed (left pending into the loop, it
  // makes the compiler wait for all memory traffic at its first use)
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // ---- producer side ------------------------------------------------------------
  // raw q/k rows of one chunk in registers, in the order stage_rows_lds_swz
  // lays them out (instruction i = pw + NP j: rows i RPI + lane / LPR, lane l
  // holds the bytes that land at 1024 i + 16 l); rows past the end are row 0.
  // pre_alpha: alpha of token `lane` (clamped to the chunk); every producer
  // loads it, producer 0 scans it.
  // The same registers carry the chain's U' of the next chunk and the
  // producers' raw rows of the chunk after it (live across a whole chunk on
  // either side): carry[j] = k rows, carry[RI + j] = q rows; chain: U' tile
  // (sl, ct) at carry[4 sl + ct].

  static_assert(2 * RI == 4 * SPW, "one carry array fits both roles");
  i32x4 carry[2 * RI];
  float pre_alpha = 1.f;
  auto fetch_raw = [&](int ch) __attribute__((always_inline)) {
    const int n = chunk_len(ch);
    const int64_t tok0 = item.tok_begin + (int64_t)ch * C;
    const int64_t row0 = (tok0 * a.H + h) * D;
    const uint16_t* kb = static_cast<const uint16_t*>(a.k) + row0;
    const uint16_t* qb = static_cast<const uint16_t*>(a.q) + row0;
#pragma unroll
    for (int j = 0; j < RI; ++j) {
      const int i = pw + NP * j;
      const int row = i * RPI + lane / LPR;
      const uint32_t off = (uint32_t)(row < n ? row : 0) * HDu + 8u * (uint32_t)((lane % LPR) ^ raw_swz<D>(row));
      carry[j] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(kb + off));
      carry[RI + j] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(qb + off));
    }
    // loads in this form are unconditional, with clamped addresses (the
    // rows past the end are masked where they are used): a load under a lane
    // mask, or a select right after one, makes the compiler wait there for
    // every load in flight
    pre_alpha = a.alpha[(tok0 + min(lane, n - 1)) * a.H + h];
  };
  auto put_raw = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < RI; ++j) {
      const int i = pw + NP * j;
      *reinterpret_cast<i32x4*>(rawK + 1024 * i + 16 * lane) = carry[j];
      *reinterpret_cast<i32x4*>(rawQ + 1024 * i + 16 * lane) = carry[RI + j];
    }
  };
  // P1: cumulative log2 decay of the staged chunk (n tokens; producer 0) into
  // buffer b
  auto p1 = [&](int b, int n) __attribute__((always_inline)) {
    if (pw == 0) {
      float* gs = reinterpret_cast<float*>(smem + b * P::BUF + P::GS);
      const float gcum = wave_inclusive_scan(log2_hw(lane < n ? pre_alpha : 1.f), lane);
      const float gl = __shfl(gcum, C - 1);
      const float gam = exp2_hw(gl);
      gs[lane] = gcum;
      gs[C + lane] = exp2_hw(gcum);
      gs[2 * C + lane] = exp2_hw(gl - gcum);
#pragma unroll
      for (int k0 = 0; k0 < D; k0 += 64) gs[3 * C + k0 + lane] = gam;
    }
  };
  // P2: Q~ and K~^T of the staged chunk into buffer b
  auto p2 = [&](int b, int n) __attribute__((always_inline)) {
    unsigned char* buf = smem + b * P::BUF;
    _Float16* sQt = reinterpret_cast<_Float16*>(buf + P::QT);
    _Float16* sKtT = reinterpret_cast<_Float16*>(buf + P::KTT);
    const float* sDec = reinterpret_cast<const float*>(buf + P::GS) + C;
    const float* sRem = sDec + C;
#pragma unroll
    for (int j = 0; j < GPT; ++j) {
      const int gi = ptid + j * NPT;
      const int c = gi / (D / 8), k8 = gi % (D / 8);
      float kx[8], qx[8];
      bf16x8_to_f32(raw_chunk<D>(rawK, c, k8, c < n), kx);
      bf16x8_to_f32(raw_chunk<D>(rawQ, c, k8, c < n), qx);
      const float dec = sDec[c], rem = sRem[c];
      f16x8 qt;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = 8 * k8 + e;
        qt[e] = (_Float16)(qx[e] * dec);
        sKtT[kk * L::LDT + swz(kk, c)] = (_Float16)(kx[e] * rem);
      }
      *reinterpret_cast<f16x8*>(sQt + c * L::LDQ + 8 * k8) = qt;
    }
  };
  // P3: the lower tiles of B = tril_incl(Q K^T) with the decay, into buffer b
  // (upper tiles stay zero from the start); the four-wavefront run schedule
  auto p3 = [&](int b, int n) __attribute__((always_inline)) {
    unsigned char* buf = smem + b * P::BUF;
    _Float16* sB = reinterpret_cast<_Float16*>(buf + P::BG);
    const float* sGs = reinterpret_cast<const float*>(buf + P::GS);
#pragma unroll
    for (int run = 0; run < 2; ++run) {
      int R, I0, I1;
      if (!gram_run<NP, false>(pw, run, R, I0, I1)) break;
      const int r = 16 * R + l16;
      bf16x8 qr[D / 32];
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) qr[ks] = as_bf16x8(raw_chunk<D>(rawQ, r, 4 * ks + g, r < n));
      const float gr = sGs[r];
      for (int I = I0; I <= I1; ++I) {
        f32x4 accB = {0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          const int i = 16 * I + l16;
          accB = mfma_bf16(as_bf16x8(raw_chunk<D>(rawK, i, 4 * ks + g, i < n)), qr[ks], accB);
        }
        const int i0 = 16 * I + 4 * g;
        const f32x4 gi = *reinterpret_cast<const f32x4*>(sGs + i0);
        f16x4 bv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float f = exp2_hw(fminf(gr - gi[e], 0.f));
          bv[e] = (_Float16)((i0 + e <= r) ? accB[e] * f : 0.f);
        }
        *reinterpret_cast<f16x4*>(sB + r * L::LDT + i0) = bv;
      }
    }
  };
  // stored W of chunk ch: producers, through registers
  constexpr int W_VEC = W_BYTES / 16;
  constexpr int W_PER_T = (W_VEC + NPT - 1) / NPT;
  f32x4 wreg[W_PER_T];
  auto fetch_w = [&](int ch) __attribute__((always_inline)) {
    const f32x4* rec = reinterpret_cast<const f32x4*>(wu_base + (int64_t)ch * WU_BYTES);
#pragma unroll
    for (int j = 0; j < W_PER_T; ++j) wreg[j] = __builtin_nontemporal_load(rec + min(ptid + j * NPT, W_VEC - 1));
  };
  auto put_w = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < W_PER_T; ++j) {
      const int e = ptid + j * NPT;
      if (e < W_VEC) reinterpret_cast<f32x4*>(sW)[e] = wreg[j];
    }
  };
  // output-gate logits of chunk ch (fused back end): rows as the raw rows,
  // into registers, then into LDS for the chain (rows past the end repeat the last)
  [[maybe_unused]] i32x4 greg[EPI != EPI_O ? RI : 1];
  [[maybe_unused]] auto fetch_g = [&](int ch) __attribute__((always_inline)) {
    const int n = chunk_len(ch);
    const uint16_t* gb = static_cast<const uint16_t*>(a.g_logit) + ((item.tok_begin + (int64_t)ch * C) * a.H + h) * D;
#pragma unroll
    for (int j = 0; j < RI; ++j) {
      const int row = (pw + NP * j) * RPI + lane / LPR;
      greg[j] = *reinterpret_cast<const i32x4*>(gb + (uint32_t)min(row, n - 1) * HDu + 8u * (uint32_t)(lane % LPR));
    }
  };
  [[maybe_unused]] auto put_g = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < RI; ++j) {
      const int row = (pw + NP * j) * RPI + lane / LPR;
      *reinterpret_cast<i32x4*>(sG + row * P::LDG + 16 * (lane % LPR)) = greg[j];
    }
  };
  // bf16 output rows of chunk chp (np tokens) from LDS, where the chain left
  // them: whole rows, 16 bytes a lane; rows past the end repeat the last one
  // (same bytes), and with real false everything goes to the sink
  [[maybe_unused]] auto store_out = [&](int chp, int np, bool real) __attribute__((always_inline)) {
    const int64_t tb = item.tok_begin + (int64_t)chp * C;
#pragma unroll
    for (int j = 0; j < RI; ++j) {
      const int row = min((pw + NP * j) * RPI + lane / LPR, np - 1);
      const i32x4 v = *reinterpret_cast<const i32x4*>(sG + row * P::LDG + 16 * (lane % LPR));
      uint16_t* dst = real ? static_cast<uint16_t*>(a.out) + ((tb + row) * a.H + h) * D + 8 * (lane % LPR)
                           : static_cast<uint16_t*>(a.out_sink);
      __builtin_nontemporal_store(v, reinterpret_cast<i32x4*>(dst));
    }
  };
  // ---- chain side: stored U' of chunk ch (this wavefront's slices) -------------
  auto fetch_up = [&](int ch) __attribute__((always_inline)) {
    const i32x4* up = reinterpret_cast<const i32x4*>(wu_base + (int64_t)ch * WU_BYTES + W_BYTES);
#pragma unroll
    for (int sl = 0; sl < SPW; ++sl)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) carry[4 * sl + ct] = __builtin_nontemporal_load(up + ((SPW * wave + sl) * 4 + ct) * 64 + lane);
  };

  // The two roles run separate loops (each holds only its own operands in
  // registers), with the same barriers: two in the prologue, two a chunk.
  // Every fetch and every put is unconditional (past the last chunk they
  // repeat it): a load or a store under a branch makes the compiler wait for
  // all memory traffic in flight where the paths join.
  const int last = n_chunks - 1;
  if (chain) {
    // fused back end: the chunk's O tiles, held from interval B into the next
    // interval A, where every chain wavefront's share of each row's sum of
    // squares is in LDS and the back end runs between that interval's products
    [[maybe_unused]] f32x4 Oh[EPI != EPI_O ? 4 : 1][SPW] = {};   // (read by the first chunk's back end,
                                                                 // whose rows go to the sink)
    // fused back end of one 16-token tile ct of a chunk whose outputs start at
    // element eb and hold n tokens: out = o rsqrt(mean o^2 + eps) norm_w sigmoid(g)
    [[maybe_unused]] auto epi_tile = [&](int ct, int64_t eb, int n) __attribute__((always_inline)) {
      const float* nw = sNw + 16 * SPW * wave + 4 * g;
      const int c = 16 * ct + l16;
      const f32x4 pp = *reinterpret_cast<const f32x4*>(sPart + 4 * c);
      const float ss = (pp[0] + pp[1]) + (pp[2] + pp[3]);
      const float r = __builtin_amdgcn_rsqf(ss / D + a.eps);
#pragma unroll
      for (int sl = 0; sl < SPW; ++sl) {
        const f32x4 w4 = *reinterpret_cast<const f32x4*>(nw + 16 * sl);
        const u32x2 gb = *reinterpret_cast<const u32x2*>(sG + c * P::LDG + 2 * (16 * SPW * wave + 16 * sl + 4 * g));
        const float gv[4] = {bf16_bits_to_f32(gb[0] & 0xFFFFu), bf16_bits_to_f32(gb[0] >> 16),
                             bf16_bits_to_f32(gb[1] & 0xFFFFu), bf16_bits_to_f32(gb[1] >> 16)};
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = Oh[ct][sl][e] * r * w4[e] * sigmoid_rcp(gv[e]);
        if constexpr (EPI == EPI_BF16) {
          // in place of the logits just read; the producers store whole rows
          *reinterpret_cast<u32x2*>(sG + c * P::LDG + 2 * (16 * SPW * wave + 16 * sl + 4 * g)) =
              u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        } else {
          // unconditional stores (rows past the end go to the sink): a store
          // under a lane mask makes the waits of interval A drain these stores
          const int64_t off = eb + (int64_t)c * HD + 16 * sl;
          float* dst = c < n ? static_cast<float*>(a.out) + off : static_cast<float*>(a.out_sink);
          *reinterpret_cast<f32x4*>(dst) = y;
        }
      }
    };
    fetch_up(0);
    __syncthreads();                             // the producers' prologue
    __syncthreads();
    // fused back end: U'(0) has landed before the loop (vmcnt(0)), so at the
    // loop head both ways in agree that U' is complete, and interval A waits
    // for none of the back end's memory traffic
    if constexpr (EPI != EPI_O) __builtin_amdgcn_s_waitcnt(0x0F70);
    for (int ch = 0; ch < n_chunks; ++ch) {
      const int b = ch & 1;
      const int64_t tok0 = item.tok_begin + (int64_t)ch * C;
      const int n = chunk_len(ch);
      refresh();
      // ---- interval A: U = U' - W S0^T (W (-S0^T) accumulated into U' directly)
      f16x8 sop[SPW][D / 32], uh[SPW][2], ul[SPW][2];
      {
        f32x4 U[SPW][4];
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl)
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) U[sl][ct] = __builtin_bit_cast(f32x4, carry[4 * sl + ct]);
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl)
#pragma unroll
          for (int ks = 0; ks < D / 32; ++ks) sop[sl][ks] = pack_perm(ST[sl][2 * ks], ST[sl][2 * ks + 1]);
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          f16x8 w[4], nsop[SPW];
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) w[ct] = ld_perm(sW, L::LDQ, 16 * ct, 32 * ks, lane);
#pragma unroll
          for (int sl = 0; sl < SPW; ++sl) nsop[sl] = -sop[sl][ks];
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int sl = 0; sl < SPW; ++sl) U[sl][ct] = mfma_f16(w[ct], nsop[sl], U[sl][ct]);
          // fused back end of the previous chunk (a full one), tile ks, between
          // these products (at the first chunk every row goes to the sink)
          if constexpr (EPI != EPI_O)
            epi_tile(ks, (tok0 - C) * HD + (int64_t)h * D + 16 * SPW * wave + 4 * g, ch > 0 ? C : 0);
        }
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) split_perm(U[sl][2 * ks], U[sl][2 * ks + 1], uh[sl][ks], ul[sl][ks]);
      }
      __syncthreads();
      // ---- interval B: O and the state update of chunk ch -------------------------
      // U' of the next chunk is fetched first: the o stores then come after
      // it, and interval A's wait for it does not wait for them
      fetch_up(min(ch + 1, last));
      const int64_t obase = tok0 * HD + (int64_t)h * D + 16 * SPW * wave + 4 * g;
      const _Float16* sQt = reinterpret_cast<const _Float16*>(smem + b * P::BUF + P::QT);
      const _Float16* sKtT = reinterpret_cast<const _Float16*>(smem + b * P::BUF + P::KTT);
      const _Float16* sB = reinterpret_cast<const _Float16*>(smem + b * P::BUF + P::BG);
      const float* sGam = reinterpret_cast<const float*>(smem + b * P::BUF + P::GS) + 3 * C;
      // O^T = S0 Q~^T + U^T B^T, one 16-token tile at a time; lane (g, l16)
      // holds O[token 16ct + l16][values 16 slice + 4g .. +3]
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        f16x8 qa[D / 32], ba[2];
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) qa[ks] = ld_perm(sQt, L::LDQ, 16 * ct, 32 * ks, lane);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) ba[ks] = ld_perm(sB, L::LDT, 16 * ct, 32 * ks, lane);
        f32x4 OT[SPW];
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl) OT[sl] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
          for (int sl = 0; sl < SPW; ++sl) OT[sl] = mfma_f16(sop[sl][ks], qa[ks], OT[sl]);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int sl = 0; sl < SPW; ++sl) {
            OT[sl] = mfma_f16(uh[sl][ks], ba[ks], OT[sl]);
            OT[sl] = mfma_f16(ul[sl][ks], ba[ks], OT[sl]);
          }
        const int c = 16 * ct + l16;
        if constexpr (EPI == EPI_O) {
          if (c < n) {
            float* orow = a.o + obase + (int64_t)c * HD;
#pragma unroll
            for (int sl = 0; sl < SPW; ++sl)
              __builtin_nontemporal_store(OT[sl], reinterpret_cast<f32x4*>(orow + 16 * sl));
          }
        } else {
          // this wavefront's share of row c's sum of squares, formed as the
          // back end's 16 lanes of 8 values form it: lane group g holds values
          // 4g .. 4g+3 of each 16-value slice, so an odd group continues its
          // even neighbour's running sum (the first four of a lane's eight), and
          // the pairwise sums over lanes, then slices, follow the xor order
          float part = 0.f;
#pragma unroll
          for (int sl = 0; sl < SPW; ++sl) {
            float s0 = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) s0 = __builtin_fmaf(OT[sl][e], OT[sl][e], s0);
            // lane groups 1 and 3 take the running sums of groups 0 and 2
            // (v_permlane16_swap: odd rows of the first operand come from the
            // even rows of the second)
            float s1 = __uint_as_float(
                __builtin_amdgcn_permlane16_swap(__float_as_uint(s0), __float_as_uint(s0), false, false)[0]);
#pragma unroll
            for (int e = 0; e < 4; ++e) s1 = __builtin_fmaf(OT[sl][e], OT[sl][e], s1);
            // groups g and g ^ 2 add their sums (v_permlane32_swap exchanges the halves)
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(s1), __float_as_uint(s1), false, false);
            s1 = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            part = sl == 0 ? s1 : part + s1;
            Oh[ct][sl] = OT[sl];
          }
          sPart[(g & 1) ? 4 * c + wave : 4 * C + lane] = part;
        }
      }
      // S^T <- 2^(G_n) S^T + K~^T U, four row tiles per batch
#pragma unroll
      for (int kb = 0; kb < KT; kb += 4) {
        f16x8 ka[4][2];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) ka[t][ks] = ld_perm_swz(sKtT, L::LDT, 16 * (kb + t), 32 * ks, lane);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const f32x4 gam = *reinterpret_cast<const f32x4*>(sGam + 16 * (kb + t) + 4 * g);
#pragma unroll
          for (int sl = 0; sl < SPW; ++sl) ST[sl][kb + t] *= gam;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int sl = 0; sl < SPW; ++sl) {
              ST[sl][kb + t] = mfma_f16(ka[t][ks], uh[sl][ks], ST[sl][kb + t]);
              ST[sl][kb + t] = mfma_f16(ka[t][ks], ul[sl][ks], ST[sl][kb + t]);
            }
        }
      }
      // snapshot after this chunk if the sequence position is a multiple of the interval
      if (a.interval > 0) {
        const int64_t pos = item.tok_in_seq + (int64_t)ch * C + n;
        if (pos % a.interval == 0) {
          const int64_t slot = item.snap_base + pos / a.interval - 1;
          float* dst = a.snapshots + (slot * a.H + h) * DD;
#pragma unroll
          for (int sl = 0; sl < SPW; ++sl)
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
              *reinterpret_cast<f32x4*>(dst + (16 * (SPW * wave + sl) + l16) * D + 16 * kt + 4 * g) = ST[sl][kt];
        }
      }
      __syncthreads();
    }
    if constexpr (EPI != EPI_O) {
      // fused back end of the last chunk
      const int64_t tl = item.tok_begin + (int64_t)last * C;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) epi_tile(ct, tl * HD + (int64_t)h * D + 16 * SPW * wave + 4 * g, chunk_len(last));
    }
    if constexpr (EPI == EPI_BF16) __syncthreads();    // the producers store the last chunk's rows
    if (item.seg == item.n_segs - 1) {
      float* dst = a.final_state + ((int64_t)item.seq * a.H + h) * DD;
#pragma unroll
      for (int sl = 0; sl < SPW; ++sl)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
          *reinterpret_cast<f32x4*>(dst + (16 * (SPW * wave + sl) + l16) * D + 16 * kt + 4 * g) = ST[sl][kt];
    }
    return;
  }

  // ---- producers: prologue (chunk 0's operands in buffer 0, W(0) in LDS) ---------
  fetch_raw(0);
  fetch_w(0);
  if constexpr (EPI != EPI_O) {
    fetch_g(0);
    for (int e = ptid; e < D; e += NPT) sNw[e] = a.norm_w[e];
  }
  for (int e = ptid; e < 2 * 6 * 256; e += NPT) {     // upper tiles of both B buffers
    const int bb = e / (6 * 256), t = (e / 256) % 6, rr = (e % 256) / 16, cc = e % 16;
    const int R = t < 3 ? 0 : (t < 5 ? 1 : 2);
    const int I = t < 3 ? t + 1 : (t < 5 ? t - 1 : 3);
    reinterpret_cast<_Float16*>(smem + bb * P::BUF + P::BG)[(16 * R + rr) * L::LDT + 16 * I + cc] = (_Float16)0.f;
  }
  put_raw();
  p1(0, chunk_len(0));
  __syncthreads();
  refresh();
  fetch_raw(min(1, last));
  p2(0, chunk_len(0));
  p3(0, chunk_len(0));
  put_w();
  __syncthreads();
  for (int ch = 0; ch < n_chunks; ++ch) {
    const int nb = (ch & 1) ^ 1;
    const bool has_next = ch + 1 < n_chunks;
    refresh();
    // ---- interval A: chunk ch+1's raw rows into LDS, its decay scan, the fetch of its W
    // (and of chunk ch's output-gate logits)
    put_raw();
    if (has_next) p1(nb, chunk_len(ch + 1));
    fetch_w(min(ch + 1, last));
    __syncthreads();
    // ---- interval B: Q~ and K~^T of ch+1, the fetch of ch+2's raw rows, B of
    // ch+1, W of ch+1 into LDS (the chain read chunk ch's in interval A)
    refresh();
    if (has_next) p2(nb, chunk_len(ch + 1));
    fetch_raw(min(ch + 2, last));
    if (has_next) p3(nb, chunk_len(ch + 1));
    put_w();
    if constexpr (EPI == EPI_BF16) store_out(ch - 1, C, ch > 0);   // chunk ch-1's rows (full), then
    if constexpr (EPI != EPI_O) {                                  // chunk ch's logits in their place
      put_g();
      fetch_g(min(ch + 1, last));
    }
    __syncthreads();
  }
  if constexpr (EPI == EPI_BF16) {
    __syncthreads();                             // the chain's back end of the last chunk
    store_out(last, chunk_len(last), true);
  }
}

// Segment scan: for every segmented sequence, head and block of 16 state rows,
// S_{s+1} = S_s M_s + N_s for s = 0 .. n_segs-2 in fp32, from S_0 = the initial
// state (or zeros); S_s is stored as the start state of segment s (S_0
// included). Rows of S evolve independently. Four wavefronts; wavefront w forms
// output columns [w D/4, (w+1) D/4) as 16x16 fp32 MFMA tiles (K = D in steps
// of 4), with S_s as the A operand and M_s as the B operand, both from LDS: M
// rows padded to D + 16 floats and S rows to D + 4, so that the four k rows
// and the sixteen state rows a K-step reads fall on distinct banks. M_{s+1}
// and N_{s+1} are fetched into registers while step s runs.
template <int D>
__global__ __launch_bounds__(256) void segment_scan_kernel(PrefillArgs a) {
  constexpr int RB = 16;                        // rows per workgroup
  constexpr int LDM = D + 16, LDSS = D + 4;     // LDS row strides (floats) of M and S
  constexpr int TPW = D / 64;                   // 16-column output tiles per wavefront
  constexpr int MV = D * D / 4 / 256;           // 16-byte pieces of M per thread
  extern __shared__ __align__(16) unsigned char smem[];
  float* sM = reinterpret_cast<float*>(smem);   // [D][LDM]
  float* sS = sM + D * LDM;                     // [RB][LDSS]
  const int nrb = D / RB;
  const int n = blockIdx.x / (a.H * nrb);
  const int rem = blockIdx.x % (a.H * nrb);
  const int h = rem / nrb, rb = rem % nrb;
  const int first = a.one_seq ? 0 : a.seq_first_item[n];
  const int ns = work_item(a, first).n_segs;
  if (ns <= 1) return;
  const int64_t DD = (int64_t)D * D;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, g = lane >> 4, l16 = lane & 15;
  {
    const float* S0 = a.init ? a.init + ((int64_t)n * a.H + h) * DD + (int64_t)rb * RB * D : nullptr;
    float* out0 = a.seg_states + ((int64_t)first * a.H + h) * DD + (int64_t)rb * RB * D;
    for (int e = tid; e < RB * D; e += 256) {
      const float x = S0 ? S0[e] : 0.f;
      sS[(e / D) * LDSS + e % D] = x;
      out0[e] = x;
    }
  }
  // M_s (all D x D) and this block's rows of N_s in the accumulator layout:
  // lane (g, l16) of wavefront w holds rows 4g + i, column w D/4 + 16t + l16
  f32x4 mreg[MV], nreg[TPW];
  auto fetch = [&](int seg) {
    const float* M = a.seg_maps + ((int64_t)(first + seg) * a.H + h) * 2 * DD;
#pragma unroll
    for (int j = 0; j < MV; ++j) mreg[j] = reinterpret_cast<const f32x4*>(M)[tid + 256 * j];
    const float* Nm = M + DD + (int64_t)rb * RB * D;
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) nreg[t][i] = Nm[(4 * g + i) * D + (D / 4) * wave + 16 * t + l16];
  };
  auto put_M = [&]() {
#pragma unroll
    for (int j = 0; j < MV; ++j) {
      const int e = 4 * (tid + 256 * j);          // element (e / D, e % D) of M
      *reinterpret_cast<f32x4*>(sM + (e / D) * LDM + e % D) = mreg[j];
    }
  };
  fetch(0);
  put_M();
  __syncthreads();
  for (int s = 0; s <= ns - 2; ++s) {
    f32x4 nadd[TPW];                              // N_s, added after the products
#pragma unroll
    for (int t = 0; t < TPW; ++t) nadd[t] = nreg[t];
    if (s + 1 <= ns - 2) fetch(s + 1);            // in flight during this step
    f32x4 acc[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) acc[t] = f32x4{0, 0, 0, 0};
#pragma unroll 8
    for (int ks = 0; ks < D / 4; ++ks) {
      const float av = sS[l16 * LDSS + 4 * ks + g];
#pragma unroll
      for (int t = 0; t < TPW; ++t)
        acc[t] = mfma_f32(av, sM[(4 * ks + g) * LDM + (D / 4) * wave + 16 * t + l16], acc[t]);
    }
    __syncthreads();                              // every wavefront is done with S_s and M_s
    float* out = a.seg_states + ((int64_t)(first + s + 1) * a.H + h) * DD + (int64_t)rb * RB * D;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int col = (D / 4) * wave + 16 * t + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = acc[t][i] + nadd[t][i];
        sS[(4 * g + i) * LDSS + col] = x;
        out[(4 * g + i) * D + col] = x;
      }
    }
    if (s + 1 <= ns - 2) put_M();
    __syncthreads();
  }
}

// Work table. Unsegmented: one item per sequence, longest first (ties keep
// sequence order) for packs of up to kSortMax sequences, sequence order
// beyond. Segmented: each sequence is cut into runs of seg_chunks chunks,
// items in sequence then segment order, with each sequence's first item
// recorded. Every item carries the first snapshot slot of its sequence.
// A single workgroup of 1024 threads; lengths come from the device copy of
// cu_seqlens. The longest-first order is a bitonic sort in LDS of the keys
// (~len << 32 | n), O(N log^2 N) over the workgroup.
constexpr int kSortMax = 8192;
__global__ __launch_bounds__(1024) void build_items_kernel(PrefillArgs a) {
  constexpr int NT = 1024;
  extern __shared__ __align__(16) unsigned char smem[];
  int64_t* snap_base = reinterpret_cast<int64_t*>(smem);                // [kSortMax] (sorted plans)
  uint64_t* keys = reinterpret_cast<uint64_t*>(smem + kSortMax * 8);    // [kSortMax]
  __shared__ int64_t carry_snap;
  __shared__ int32_t carry_items;
  __shared__ int64_t part_snap[NT];
  __shared__ int32_t part_items[NT];
  const int32_t N = a.num_seqs;
  const int64_t* cu = a.cu_dev;
  const int64_t seg_tokens = (int64_t)a.seg_chunks * C;
  const bool sorted = a.seg_chunks == 0 && N <= kSortMax;
  const int tid = threadIdx.x;
  if (tid == 0) { carry_snap = 0; carry_items = 0; }
  __syncthreads();
  // prefix sums over sequences (snapshot slots, items) in blocks of NT
  for (int32_t base = 0; base < N; base += NT) {
    const int32_t n = base + tid;
    const int64_t len = n < N ? cu[n + 1] - cu[n] : 0;
    const int64_t ns = (n < N && a.interval > 0) ? len / a.interval : 0;
    int32_t nseg = n < N ? 1 : 0;
    if (n < N && seg_tokens > 0 && len > seg_tokens) nseg = (int32_t)((len + seg_tokens - 1) / seg_tokens);
    part_snap[tid] = ns;
    part_items[tid] = nseg;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
      const int64_t ys = tid >= off ? part_snap[tid - off] : 0;
      const int32_t yi = tid >= off ? part_items[tid - off] : 0;
      __syncthreads();
      part_snap[tid] += ys;
      part_items[tid] += yi;
      __syncthreads();
    }
    if (n < N) {
      const int64_t sb = carry_snap + part_snap[tid] - ns;
      const int32_t first = carry_items + part_items[tid] - nseg;
      if (sorted) {
        snap_base[n] = sb;
        keys[n] = ((uint64_t)(~(uint32_t)len) << 32) | (uint32_t)n;   // ascending: longest first
      } else if (a.seg_chunks == 0) {
        PrefillItem it;
        it.tok_begin = cu[n];
        it.tok_in_seq = 0;
        it.snap_base = sb;
        it.n_tokens = (int32_t)len;
        it.seq = n;
        it.seg = 0;
        it.n_segs = 1;
        a.items[n] = it;
      } else {
        a.seq_first_item[n] = first;
        for (int32_t sg = 0; sg < nseg; ++sg) {
          PrefillItem it;
          it.tok_in_seq = (int64_t)sg * seg_tokens;
          it.tok_begin = cu[n] + it.tok_in_seq;
          it.snap_base = sb;
          it.n_tokens = (int32_t)(nseg == 1 ? len : min(seg_tokens, len - it.tok_in_seq));
          it.seq = n;
          it.seg = sg;
          it.n_segs = nseg;
          a.items[first + sg] = it;
        }
      }
    }
    __syncthreads();
    if (tid == NT - 1) {
      carry_snap += part_snap[NT - 1];
      carry_items += part_items[NT - 1];
    }
    __syncthreads();
  }
  if (!sorted) return;                           // (uniform)
  // bitonic sort of the keys, padded to a power of two with the largest key
  int P = 1;
  while (P < N) P <<= 1;
  for (int e = N + tid; e < P; e += NT) keys[e] = ~(uint64_t)0;
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int e = tid; e < P; e += NT) {
        const int f = e ^ j;
        if (f > e) {
          const uint64_t x = keys[e], y = keys[f];
          const bool up = (e & k) == 0;
          if ((x > y) == up) { keys[e] = y; keys[f] = x; }
        }
      }
      __syncthreads();
    }
  }
  for (int p = tid; p < N; p += NT) {
    const int32_t n = (int32_t)(keys[p] & 0xFFFFFFFFu);
    PrefillItem it;
    it.tok_begin = cu[n];
    it.tok_in_seq = 0;
    it.snap_base = snap_base[n];
    it.n_tokens = (int32_t)(cu[n + 1] - cu[n]);
    it.seq = n;
    it.seg = 0;
    it.n_segs = 1;
    a.items[p] = it;
  }
}

template <int D, bool BF16, bool PK, bool MAP, bool WU, int EPI = EPI_O>
hipError_t launch_pass(const PrefillArgs& a, hipStream_t s) {
  using L = Lds<D>;
  constexpr int lds = EPI == EPI_O ? L::TOTAL : L::TOTAL_EPI;
  static_assert(lds <= 160 * 1024, "LDS budget");
  constexpr int NT = 64 * waves_for<D>();
  auto kern = prefill_kernel<D, BF16, PK, MAP, WU, waves_for<D>(), EPI>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.n_items * a.H), dim3(NT), lds, s, a);
  return hipGetLastError();
}

template <int D, int EPI>
hipError_t launch_wu_pipe(const PrefillArgs& a, hipStream_t s) {
  using P = LdsPipe<D>;
  constexpr int lds = EPI == EPI_O ? P::TOTAL : P::TOTAL_EPI;
  static_assert(lds <= 160 * 1024, "LDS budget");
  auto kern = prefill_wu_pipe_kernel<D, EPI>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.n_items * a.H), dim3(512), lds, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_map_chain(const PrefillArgs& a, hipStream_t s) {
  using P = LdsMapChain<D>;
  static_assert(P::TOTAL <= 160 * 1024, "LDS budget");
  auto kern = prefill_map_chain_kernel<D>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, P::TOTAL);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.n_items * a.H), dim3(768), P::TOTAL, s, a);
  return hipGetLastError();
}

template <int D, bool BF16, bool PK>
hipError_t launch_t(const PrefillArgs& a, hipStream_t s) {
  // fused back end: split sequences only (a whole pass may still run, for
  // empty sequences' final states, and writes no o)
  if (a.out != nullptr && a.seg_chunks == 0) return hipErrorInvalidValue;
  if (a.seg_chunks == 0) return launch_pass<D, BF16, PK, false, false>(a, s);
  hipError_t e;                                                 // pass 1: segment maps, W and U' per chunk
  if constexpr (D == 128 && BF16 && !PK)
    e = launch_map_chain<D>(a, s);
  else
    e = launch_pass<D, BF16, PK, true, false>(a, s);
  if (e != hipSuccess) return e;
  constexpr int scan_lds = (D * (D + 16) + 16 * (D + 4)) * 4;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(segment_scan_kernel<D>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, scan_lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(segment_scan_kernel<D>, dim3(a.num_seqs * a.H * (D / 16)), dim3(256), scan_lds, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (D == 128 && BF16 && !PK) {                      // pass 3: every segment (qk_shift is 0 at d = 128)
    if (a.out == nullptr) e = launch_wu_pipe<D, EPI_O>(a, s);
    else if (a.out_bf16) e = launch_wu_pipe<D, EPI_BF16>(a, s);
    else e = launch_wu_pipe<D, EPI_F32>(a, s);
  } else if (a.out == nullptr) {
    e = launch_pass<D, BF16, PK, false, true>(a, s);
  } else if constexpr (D == 64 && BF16 && PK) {                 // the KDA layer's form
    e = a.out_bf16 ? launch_pass<D, BF16, PK, false, true, EPI_BF16>(a, s)
                   : launch_pass<D, BF16, PK, false, true, EPI_F32>(a, s);
  } else {
    return hipErrorInvalidValue;                                  // no fused back end in this form
  }
  if (e != hipSuccess || !a.any_whole) return e;
  return launch_pass<D, BF16, PK, false, false>(a, s);          // sequences that are not split
}

// Row copy with zero fill (see launch_copy_rows): one piece (16 or 4 bytes)
// per thread, blockIdx.y over rows in steps of 65535.
template <class T>
__global__ __launch_bounds__(256) void copy_rows_kernel(const T* src, T* dst, int64_t n_rows, int64_t src_stride,
                                                        int64_t dst_stride, int64_t copy, int64_t fill) {
  const int64_t piece = (int64_t)blockIdx.x * 256 + threadIdx.x;   // piece within the row
  if (piece >= copy + fill) return;
  for (int64_t r = blockIdx.y; r < n_rows; r += gridDim.y) {
    T* d = dst + r * dst_stride + piece;
    if (piece < copy) *d = src[r * src_stride + piece];
    else *d = T{};
  }
}

}  // namespace

hipError_t launch_copy_rows(const void* src, void* dst, int64_t n_rows, int64_t src_stride, int64_t dst_stride,
                            int64_t copy, int64_t fill, hipStream_t s) {
  if (n_rows <= 0 || copy + fill <= 0) return hipSuccess;
  const uintptr_t all = reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst) |
                        (uintptr_t)src_stride | (uintptr_t)dst_stride | (uintptr_t)copy | (uintptr_t)fill;
  const int unit = (all & 15) == 0 ? 16 : 4;        // 16-byte pieces where everything allows
  const int64_t pieces = (copy + fill) / unit;
  const dim3 grid((unsigned)((pieces + 255) / 256), (unsigned)(n_rows < 65535 ? n_rows : 65535));
  if (unit == 16)
    hipLaunchKernelGGL(copy_rows_kernel<uint4>, grid, dim3(256), 0, s, static_cast<const uint4*>(src),
                       static_cast<uint4*>(dst), n_rows, src_stride / 16, dst_stride / 16, copy / 16, fill / 16);
  else
    hipLaunchKernelGGL(copy_rows_kernel<uint32_t>, grid, dim3(256), 0, s, static_cast<const uint32_t*>(src),
                       static_cast<uint32_t*>(dst), n_rows, src_stride / 4, dst_stride / 4, copy / 4, fill / 4);
  return hipGetLastError();
}

hipError_t launch_prefill(PrefillArgs a, int d, bool bf16, bool per_key, hipStream_t s) {
  if (!a.one_seq) {                              // (one sequence: the kernels form the items)
    constexpr int items_lds = kSortMax * 16;     // snapshot bases and sort keys
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(build_items_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, items_lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(build_items_kernel, dim3(1), dim3(1024), items_lds, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (d == 64) {
    if (bf16) return per_key ? launch_t<64, true, true>(a, s) : launch_t<64, true, false>(a, s);
    return per_key ? launch_t<64, false, true>(a, s) : launch_t<64, false, false>(a, s);
  }
  if (bf16) return per_key ? launch_t<128, true, true>(a, s) : launch_t<128, true, false>(a, s);
  return per_key ? launch_t<128, false, true>(a, s) : launch_t<128, false, false>(a, s);
}

}  // namespace kda
