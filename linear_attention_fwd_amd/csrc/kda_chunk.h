// kda_chunk.h -- stages of the per-chunk prep shared by the chunk kernels.
//
// A chunk is C = 64 tokens of one head, worked on by one workgroup of four
// waves.  Thread layout of the token-parallel stages: wave w owns subtile w
// (tokens 16w..16w+15); lane (tq, cg) holds tokens 16w + 4tq + r (r = 0..3),
// channels 8cg..8cg+7.  The stages, in the order the kernels call them:
//
//   a1  prep_gate_cumsum     gate g = g_min*sigmoid(exp(A_h) z) and the
//       in-chunk inclusive cumulative log-decay G ("序列维度（下）", eq. (3),
//       eq. (5), section "数值问题"), in base-2 units;
//   a2  prep_decay_operands  the decay factors Q_decay = e^G q, K_decay =
//       e^G k, K_restore = e^(G_C - G) k and the 16-token subtile operands
//       referenced to the first token s of the query subtile: e^(G_i - G_s)
//       <= 1 on the query side, e^(G_s - G_j) < e^75 on the key side (g >
//       g_min = -5 keeps it inside the bf16 range, section "K3 的改动：下界衰减");
//   a3  prep_subtile_products  L = StrictTril(Diag(beta) K_decay K_inv^T) and
//       M_qk = Tril(Q_decay K_inv^T) (diagonal kept) per 16x16 subtile pair on
//       MFMA (SemiAnalysis page, section "FlashKDA 算法");
//   a4  prep_diag_inverse + prep_block_columns  the UT transform INV =
//       (I + L)^-1 ("序列维度（下）", section "UT 变换"): each 16x16 diagonal
//       block by repeated squaring, (I + L)^-1 = (I - L)(I + L^2)(I + L^4)(I + L^8),
//       then one block column per wave, X_IJ = -T_II sum_K L_IK X_KJ, stored as
//       INV Diag(beta).
//
// Where a stage's result goes (LDS for the fused kernel, the chunk image in
// global memory for the split prep kernel) is the caller's choice: a2 and a3
// hand their recurrence operands to a sink functor.
#pragma once
#include "kda_device.h"
#include <type_traits>
#include "kda_launch.h"

namespace kda {

constexpr int FWD_THREADS = 256;
constexpr float LOG2E = 1.4426950408889634f;

// Keep the instruction scheduler from moving work across chunk phases.
#define SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// ---------------------------------------------------------------------------
// MFMA operand plumbing for the two arithmetic modes.  Operand reads take a
// tile, a row and the 32-wide k block; lane group g reads elements
// [32kb + 8g, 32kb + 8g + 8) of the row (both operands agree on that order).
// ---------------------------------------------------------------------------
template <bool F32C> struct Arith;

template <> struct Arith<false> {  // bf16 operands, fp32 accumulate
  using E = bf16_t;
  struct BReg { bf16x8 v; };
  static __device__ __forceinline__ E cvt(float x) { return f32_to_bf16(x); }
  static __device__ __forceinline__ float tof(E x) { return bf16_to_f32(x); }
  static __device__ __forceinline__ BReg breg(floatx4 t0, floatx4 t1) {
    BReg b;
    b.v = to_bf16x8(floatx8{t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]});
    return b;
  }
  template <int COLS>
  static __device__ __forceinline__ floatx4 k32(floatx4 acc, const E *tile, int row, int kb, int g,
                                               const BReg &b) {
    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(tile + Tile<E, COLS>::idx(row, 32 * kb + 8 * g));
    return mfma_bf16_k32(a, b.v, acc);
  }
  // acc += A . B with the A operand in registers and B read from an LDS row
  template <int COLS>
  static __device__ __forceinline__ floatx4 k32_regA(floatx4 acc, const BReg &a, const E *tile, int row,
                                                    int kb, int g) {
    const bf16x8 b = *reinterpret_cast<const bf16x8 *>(tile + Tile<E, COLS>::idx(row, 32 * kb + 8 * g));
    return mfma_bf16_k32(a.v, b, acc);
  }
  template <int COLS>
  static __device__ __forceinline__ BReg breg_lds(const E *tile, int row, int kb, int g) {
    BReg b;
    b.v = *reinterpret_cast<const bf16x8 *>(tile + Tile<E, COLS>::idx(row, 32 * kb + 8 * g));
    return b;
  }
  // B operand from LDS scaled per k (sc points at the natural-order scale row)
  template <int COLS>
  static __device__ __forceinline__ BReg breg_lds_scaled(const E *tile, int row, int kb, int g,
                                                         const float *sc) {
    const bf16x8 raw = *reinterpret_cast<const bf16x8 *>(tile + Tile<E, COLS>::idx(row, 32 * kb + 8 * g));
    const float4 s0 = *reinterpret_cast<const float4 *>(sc + 32 * kb + 8 * g);
    const float4 s1 = *reinterpret_cast<const float4 *>(sc + 32 * kb + 8 * g + 4);
    const floatx8 f = __builtin_convertvector(raw, floatx8) *
                      floatx8{s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    BReg b;
    b.v = to_bf16x8(f);
    return b;
  }
  // 16x16x16 step: acc += A . B with A given row-wise (4 values of row j, k = 4g..4g+3)
  // and B in accumulator layout (4 values: rows 4g..4g+3 of column j).
  static __device__ __forceinline__ floatx4 k16(floatx4 acc, floatx4 a, floatx4 b) {
    return mfma_bf16_k16(to_bf16x4(a), to_bf16x4(b), acc);
  }
  static __device__ __forceinline__ void store4(E *p, const float *x) {  // 4 consecutive
    *reinterpret_cast<bf16x4 *>(p) = to_bf16x4(floatx4{x[0], x[1], x[2], x[3]});
  }
  static __device__ __forceinline__ floatx4 load4(const E *p) {
    const uint2 w = *reinterpret_cast<const uint2 *>(p);
    return floatx4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                   __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u)};
  }
};

template <> struct Arith<true> {  // fp32 operands, fp32 MFMA
  using E = float;
  struct BReg { float v[8]; };
  static __device__ __forceinline__ E cvt(float x) { return x; }
  static __device__ __forceinline__ float tof(E x) { return x; }
  static __device__ __forceinline__ BReg breg(floatx4 t0, floatx4 t1) {
    BReg b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      b.v[e] = t0[e];
      b.v[4 + e] = t1[e];
    }
    return b;
  }
  template <int COLS>
  static __device__ __forceinline__ floatx4 k32(floatx4 acc, const E *tile, int row, int kb, int g,
                                               const BReg &b) {
    const float4 a0 = *reinterpret_cast<const float4 *>(tile + Tile<E, COLS>::idx(row, 32 * kb + 8 * g));
    const float4 a1 = *reinterpret_cast<const float4 *>(tile + Tile<E, COLS>::idx(row, 32 * kb + 8 * g + 4));
    const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = mfma_f32_k4(a[e], b.v[e], acc);
    return acc;
  }
  template <int COLS>
  static __device__ __forceinline__ floatx4 k32_regA(floatx4 acc, const BReg &a, const E *tile, int row,
                                                    int kb, int g) {
    const float4 b0 = *reinterpret_cast<const float4 *>(tile + Tile<E, COLS>::idx(row, 32 * kb + 8 * g));
    const float4 b1 = *reinterpret_cast<const float4 *>(tile + Tile<E, COLS>::idx(row, 32 * kb + 8 * g + 4));
    const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = mfma_f32_k4(a.v[e], bv[e], acc);
    return acc;
  }
  template <int COLS>
  static __device__ __forceinline__ BReg breg_lds(const E *tile, int row, int kb, int g) {
    const float4 b0 = *reinterpret_cast<const float4 *>(tile + Tile<E, COLS>::idx(row, 32 * kb + 8 * g));
    const float4 b1 = *reinterpret_cast<const float4 *>(tile + Tile<E, COLS>::idx(row, 32 * kb + 8 * g + 4));
    BReg b = {{b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w}};
    return b;
  }
  template <int COLS>
  static __device__ __forceinline__ BReg breg_lds_scaled(const E *tile, int row, int kb, int g,
                                                         const float *sc) {
    BReg b = breg_lds<COLS>(tile, row, kb, g);
    const float4 s0 = *reinterpret_cast<const float4 *>(sc + 32 * kb + 8 * g);
    const float4 s1 = *reinterpret_cast<const float4 *>(sc + 32 * kb + 8 * g + 4);
    b.v[0] *= s0.x; b.v[1] *= s0.y; b.v[2] *= s0.z; b.v[3] *= s0.w;
    b.v[4] *= s1.x; b.v[5] *= s1.y; b.v[6] *= s1.z; b.v[7] *= s1.w;
    return b;
  }
  static __device__ __forceinline__ floatx4 k16(floatx4 acc, floatx4 a, floatx4 b) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = mfma_f32_k4(a[e], b[e], acc);
    return acc;
  }
  static __device__ __forceinline__ void store4(E *p, const float *x) {
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
  static __device__ __forceinline__ floatx4 load4(const E *p) {
    const float4 w = *reinterpret_cast<const float4 *>(p);
    return floatx4{w.x, w.y, w.z, w.w};
  }
};

// ---- document and chunk bookkeeping ----------------------------------------
// The document offsets are read through the constant address space, so that
// with a uniform index they come in by scalar loads.  Vector loads would share
// the wave's vmcnt with its copies and stores, and waiting for one of them
// would wait for all of those issued before it.
__device__ __forceinline__ int64_t cu_load(const int32_t *cu, int i) {
  return (int64_t)((const __attribute__((address_space(4))) int32_t *)cu)[i];
}
// document offsets; cu == nullptr means one document [0, T)
__device__ __forceinline__ int64_t cu_at(const int32_t *cu, int64_t T, int i) {
  return cu ? cu_load(cu, i) : (i == 0 ? (int64_t)0 : T);
}
// largest d in [0, N-1] with cu[d] <= pos (skips empty documents starting at pos)
__device__ __forceinline__ int doc_of(const int32_t *cu, int N, int64_t pos) {
  if (!cu) return 0;
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_load(cu, mid) <= pos) lo = mid; else hi = mid - 1;
  }
  return uni(lo);
}
// document owning a chunk slot (first_slot in kda_launch.h): largest d with first_slot(d) <= slot
__device__ __forceinline__ int doc_of_slot(const int32_t *cu, int N, int64_t slot) {
  if (!cu) return 0;
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (first_slot(cu_load(cu, mid), mid) <= slot) lo = mid; else hi = mid - 1;
  }
  return uni(lo);
}

// ---- LDS shared by the prep stages -------------------------------------------
struct PrepLds {
  float GC2[D];       // G_C (base 2)
  float Gref[4][D];   // G (base 2) at the first token of each subtile
  float Gend[4][D];   // G (base 2) at the last token of each subtile (unbounded gate)
  float F[6][D];      // e^(Gref[I] - Gref[J]) for I > J
  float beta[CH];
  union {
    float wtot[4][D];  // per-wave cumulative-sum totals (a1 only)
    float Fd[4][D];    // unbounded gate: e^(Gref[I] - Gend[I]), the diagonal subtiles' factor
  };
};

// Unbounded gate: diagonal subtile I takes the two-factor MFMA form of the
// bounded gate when, in every channel, its decay over the subtile G_s - G_e
// (base 2) is at most DIAG_RANGE2.  The key operand e^(G_s - G_j) k_j then
// stays below 2^116 |k_j| (no overflow) and the query operand e^(G_i - G_s) q_i
// above 2^-116 |q_i|: only query elements under 2^-10 can drop below the
// smallest normal float, in the last tokens of the widest channels, where
// their terms are under 0.1% of a unit-norm entry.  (The bounded gate's own
// range is at most 15 * 5 / ln 2 = 108.)  Wave-uniform; needs Gref and Gend
// (after prep_gate_cumsum).
constexpr float DIAG_RANGE2 = 116.0f;
__device__ __forceinline__ bool diag_two_factor(const PrepLds &ps, int I) {
  const int lane = threadIdx.x & 63;
  const float r0 = ps.Gref[I][lane] - ps.Gend[I][lane];
  const float r1 = ps.Gref[I][lane + 64] - ps.Gend[I][lane + 64];
  return __ballot(!(r0 <= DIAG_RANGE2 && r1 <= DIAG_RANGE2)) == 0;  // a NaN range fails too
}

// Raw inputs: q or k of this thread's 4 tokens (8 channels each) scaled to unit
// L2 norm per token and rounded back to bf16, the precision every matrix
// operand built from them has; the 16 lanes of a token group (lane bits 0-3)
// hold the 128 channels of its tokens.  An all-zero row (a padding row) stays
// zero.
__device__ __forceinline__ void l2norm_rows(bufio<bf16_t>::raw8 (&R)[4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float x[8];
    bufio<bf16_t>::cvt8(R[r], x);
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) ss = fmaf(x[c], x[c], ss);
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    ss += __shfl_xor(ss, 4);
    ss += __shfl_xor(ss, 8);
    const float sc = ss > 0.f ? __builtin_amdgcn_rsqf(ss) : 0.f;
    const bf16x8 y = to_bf16x8(floatx8{x[0] * sc, x[1] * sc, x[2] * sc, x[3] * sc, x[4] * sc,
                                       x[5] * sc, x[6] * sc, x[7] * sc});
    R[r].a = __builtin_bit_cast(u32x4, y);
  }
}
// The same on fp32 inputs: the rows stay in fp32 (the precision of the fp32
// build's operands).
__device__ __forceinline__ void l2norm_rows(bufio<float>::raw8 (&R)[4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float x[8];
    bufio<float>::cvt8(R[r], x);
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) ss = fmaf(x[c], x[c], ss);
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    ss += __shfl_xor(ss, 4);
    ss += __shfl_xor(ss, 8);
    const float sc = ss > 0.f ? __builtin_amdgcn_rsqf(ss) : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      R[r].a[i] = __float_as_uint(x[i] * sc);
      R[r].b[i] = __float_as_uint(x[4 + i] * sc);
    }
  }
}

// a1: gate and inclusive cumulative sum over the chunk (base 2).  Tokens at or
// beyond len are padding: no decay.  Leaves G[r][c] for this thread's tokens
// and channels, beta, Gref and GC2 in LDS (and Gend for the unbounded gate);
// ends with a barrier.  UNB selects the unbounded gate (gmin2 unused);
// beta_logit takes beta as a logit (raw inputs: beta = sigmoid(logit), fp32).
template <class IO, bool UNB = false>
__device__ __forceinline__ void prep_gate_cumsum(PrepLds &ps, const typename IO::raw8 (&Rz)[4],
                                                 typename IO::raw1 Rb, float c1, float gmin2,
                                                 int len, int tid, int w, int tq, int cg,
                                                 float (&G)[4][8], bool beta_logit = false) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const bool tok = 16 * w + 4 * tq + r < len;
    const float gm = tok ? gmin2 : 0.f;
    const float cm = tok ? c1 : 0.f;
    float zz[8];
    IO::cvt8(Rz[r], zz);
#pragma unroll
    for (int c = 0; c < 8; ++c)
      G[r][c] = UNB ? kda_gate2_softplus(zz[c], cm) : kda_gate2(zz[c], c1, gm);
  }
  if (tid < CH) {
    const float b = IO::cvt1(Rb);
    ps.beta[tid] = beta_logit ? __builtin_amdgcn_rcpf(1.0f + __expf(-b)) : b;
  }
  // in-lane over r, across the 4 token groups of the wave (lanes 16 apart),
  // then across waves
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    G[1][c] += G[0][c];
    G[2][c] += G[1][c];
    G[3][c] += G[2][c];
    const float tot = G[3][c];
    const float up16 = __shfl_up(tot, 16);
    const float x1 = tot + (tq >= 1 ? up16 : 0.f);
    const float up32 = __shfl_up(x1, 32);
    const float excl = x1 + (tq >= 2 ? up32 : 0.f) - tot;
#pragma unroll
    for (int r = 0; r < 4; ++r) G[r][c] += excl;
  }
  if (tq == 3) {
    *reinterpret_cast<float4 *>(&ps.wtot[w][8 * cg]) = make_float4(G[3][0], G[3][1], G[3][2], G[3][3]);
    *reinterpret_cast<float4 *>(&ps.wtot[w][8 * cg + 4]) = make_float4(G[3][4], G[3][5], G[3][6], G[3][7]);
  }
  __syncthreads();
  SCHED_FENCE();
  {
    const float4 t0a = *reinterpret_cast<const float4 *>(&ps.wtot[0][8 * cg]);
    const float4 t0b = *reinterpret_cast<const float4 *>(&ps.wtot[0][8 * cg + 4]);
    const float4 t1a = *reinterpret_cast<const float4 *>(&ps.wtot[1][8 * cg]);
    const float4 t1b = *reinterpret_cast<const float4 *>(&ps.wtot[1][8 * cg + 4]);
    const float4 t2a = *reinterpret_cast<const float4 *>(&ps.wtot[2][8 * cg]);
    const float4 t2b = *reinterpret_cast<const float4 *>(&ps.wtot[2][8 * cg + 4]);
    const float t0[8] = {t0a.x, t0a.y, t0a.z, t0a.w, t0b.x, t0b.y, t0b.z, t0b.w};
    const float t1[8] = {t1a.x, t1a.y, t1a.z, t1a.w, t1b.x, t1b.y, t1b.z, t1b.w};
    const float t2[8] = {t2a.x, t2a.y, t2a.z, t2a.w, t2b.x, t2b.y, t2b.z, t2b.w};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float off = (w > 0 ? t0[c] : 0.f) + (w > 1 ? t1[c] : 0.f) + (w > 2 ? t2[c] : 0.f);
#pragma unroll
      for (int r = 0; r < 4; ++r) G[r][c] += off;
    }
  }
  if (tq == 0) {
    *reinterpret_cast<float4 *>(&ps.Gref[w][8 * cg]) = make_float4(G[0][0], G[0][1], G[0][2], G[0][3]);
    *reinterpret_cast<float4 *>(&ps.Gref[w][8 * cg + 4]) = make_float4(G[0][4], G[0][5], G[0][6], G[0][7]);
  }
  if (w == 3 && tq == 3) {
    *reinterpret_cast<float4 *>(&ps.GC2[8 * cg]) = make_float4(G[3][0], G[3][1], G[3][2], G[3][3]);
    *reinterpret_cast<float4 *>(&ps.GC2[8 * cg + 4]) = make_float4(G[3][4], G[3][5], G[3][6], G[3][7]);
  }
  if (UNB && tq == 3) {
    *reinterpret_cast<float4 *>(&ps.Gend[w][8 * cg]) = make_float4(G[3][0], G[3][1], G[3][2], G[3][3]);
    *reinterpret_cast<float4 *>(&ps.Gend[w][8 * cg + 4]) = make_float4(G[3][4], G[3][5], G[3][6], G[3][7]);
  }
  __syncthreads();
  SCHED_FENCE();
}

// a2: decay factors of this thread's 4 tokens x 8 channels.  The subtile
// operands Qh and Ki go to LDS tiles (natural channel order) and Kh to
// kh_sink(r, i, kh[8]) (token 16w + 4tq + r = i); per token row i the sink
// receives K_decay and Q_decay (row_sink(i, kdec[8], qdec[8])); K_restore is
// returned for the caller to store.
//
// The query side (Qh, Kh) is referenced to the first token s of the subtile,
// e^(G_i - G_s) <= 1.  For the bounded gate the key side Ki is referenced to
// that token too, e^(G_s - G_j) < e^75 (g >= -5 per step over at most 15
// steps), so even the diagonal subtile products split into two factors
// ("序列维度（下）", section on the 16-token subtiles).  Without a lower bound
// (UNB) that factor has no bound, so the key side is referenced to the last
// token e of its subtile instead, e^(G_e - G_j) <= 1: off-diagonal pairs then
// take the factor e^(G_s(I) - G_e(J)) <= 1 and the diagonal subtiles are done
// per position (prep_diag_positions).  K_restore = e^(G_C - G_j) k_j is Ki
// times e^(G_C - G_ref), in the unbounded case a product of factors <= 1.
template <class Ar, class IO, bool UNB = false, class KhSink, class RowSink>
__device__ __forceinline__ void prep_decay_operands(const PrepLds &ps, typename Ar::E *Qh,
                                                    KhSink &&kh_sink, typename Ar::E *Ki,
                                                    const typename IO::raw8 (&Rq)[4],
                                                    const typename IO::raw8 (&Rk)[4],
                                                    const float (&G)[4][8], int w, int tq, int cg,
                                                    float (&Kres)[4][8], RowSink &&row_sink) {
  using TD = Tile<typename Ar::E, D>;
  float Pj[8], Rj[8], gref[8], gkey[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    gref[c] = ps.Gref[w][8 * cg + c];
    gkey[c] = UNB ? ps.Gend[w][8 * cg + c] : gref[c];
    Pj[c] = __builtin_amdgcn_exp2f(gref[c]);                       // e^(G_s)
    Rj[c] = __builtin_amdgcn_exp2f(ps.GC2[8 * cg + c] - gkey[c]);  // e^(G_C - G_ref) <= 1
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 16 * w + 4 * tq + r;
    float qv[8], kv[8], qh[8], kh[8], ki[8], qdec[8], kdec[8];
    IO::cvt8(Rq[r], qv);
    IO::cvt8(Rk[r], kv);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float e1 = __builtin_amdgcn_exp2f(G[r][c] - gref[c]);  // <= 1
      // bounded: 1 / e1 < e^75; unbounded: e^(G_e - G_i) <= 1
      const float e2 = UNB ? __builtin_amdgcn_exp2f(gkey[c] - G[r][c]) : __builtin_amdgcn_rcpf(e1);
      qh[c] = qv[c] * e1;
      kh[c] = kv[c] * e1;
      ki[c] = kv[c] * e2;
      qdec[c] = qh[c] * Pj[c];
      kdec[c] = kh[c] * Pj[c];
      Kres[r][c] = ki[c] * Rj[c];
    }
    Ar::store4(&Qh[TD::idx(i, 8 * cg)], qh);
    Ar::store4(&Qh[TD::idx(i, 8 * cg + 4)], qh + 4);
    kh_sink(r, i, kh);
    Ar::store4(&Ki[TD::idx(i, 8 * cg)], ki);
    Ar::store4(&Ki[TD::idx(i, 8 * cg + 4)], ki + 4);
    row_sink(i, kdec, qdec);
    SCHED_FENCE();
  }
}

// F[pair][c] = e^(Gref[I][c] - Gref[J][c]) (UNB: e^(Gref[I][c] - Gend[J][c]) <= 1),
// pairs (1,0),(2,0),(2,1),(3,0),(3,1),(3,2): moves the key side's reference to
// the first token of the query subtile.  UNB also gives the diagonal subtiles
// Fd[I][c] = e^(Gref[I][c] - Gend[I][c]) >= 1 (clamped below fp32 overflow; it
// is used only where diag_two_factor holds).  Ends before a barrier: wtot,
// which Fd overlays, is dead once prep_gate_cumsum has returned.
template <bool UNB = false>
__device__ __forceinline__ void prep_pair_factors(PrepLds &ps, int tid) {
  for (int x = tid; x < (UNB ? 10 : 6) * D; x += FWD_THREADS) {
    const int pi = x / D, c = x % D;
    if (UNB && pi >= 6) {
      ps.Fd[pi - 6][c] = __builtin_amdgcn_exp2f(fminf(ps.Gref[pi - 6][c] - ps.Gend[pi - 6][c], 126.0f));
      continue;
    }
    const int I = (pi == 0) ? 1 : (pi < 3 ? 2 : 3);
    const int J = (pi == 0) ? 0 : (pi < 3 ? pi - 1 : pi - 3);
    ps.F[pi][c] = __builtin_amdgcn_exp2f(ps.Gref[I][c] - (UNB ? ps.Gend[J][c] : ps.Gref[J][c]));
  }
}

// a3: A_qk and A_kk per subtile pair (I >= J); wave w takes pairs w, w+4, w+8.
// Products are formed transposed, (K_inv_J)(Q_I)^T, so lane (g, j) ends up
// with row j of the pair's tile at columns 4g..4g+3 and writes them at once.
// L (natural order, operand precision) goes to LDS; M_qk goes to
// mqk_sink(row, J, mq[4]).  PRODUCTS selects M_qk (1), L (2) or both (3); a
// product not selected reads nothing from its tile (Qh or Kh).  UNB: the key
// side is referenced to the end of its subtile; a diagonal pair takes the
// factor Fd where diag_two_factor holds and is left to prep_diag_positions
// otherwise.
constexpr int PROD_MQK = 1, PROD_L = 2;
template <class Ar, int PRODUCTS, bool UNB = false, class MqkSink>
__device__ __forceinline__ void prep_subtile_products(const PrepLds &ps, const typename Ar::E *Qh,
                                                      const typename Ar::E *Kh,
                                                      const typename Ar::E *Ki, typename Ar::E *L,
                                                      int w, int g, int j, MqkSink &&mqk_sink) {
  using BReg = typename Ar::BReg;
  using TL = Tile<typename Ar::E, CH>;
  for (int pidx = w; pidx < 10; pidx += 4) {
    const int I = (pidx == 0) ? 0 : (pidx < 3 ? 1 : (pidx < 6 ? 2 : 3));
    const int J = pidx - I * (I + 1) / 2;
    if (UNB && I == J && !diag_two_factor(ps, I)) continue;
    floatx4 aq = {0.f, 0.f, 0.f, 0.f}, ak = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      BReg kin;  // key side of subtile J, referenced to the first token of subtile I
      if (I == J) {
        kin = UNB ? Ar::template breg_lds_scaled<D>(Ki, 16 * J + j, kb, g, ps.Fd[I])
                  : Ar::template breg_lds<D>(Ki, 16 * J + j, kb, g);
      } else {
        const int fp = I * (I - 1) / 2 + J;
        kin = Ar::template breg_lds_scaled<D>(Ki, 16 * J + j, kb, g, ps.F[fp]);
      }
      if constexpr ((PRODUCTS & PROD_MQK) != 0) aq = Ar::template k32_regA<D>(aq, kin, Qh, 16 * I + j, kb, g);
      if constexpr ((PRODUCTS & PROD_L) != 0) ak = Ar::template k32_regA<D>(ak, kin, Kh, 16 * I + j, kb, g);
    }
    // lane (g, j): element r is (row j of subtile I, column 4g + r of subtile J)
    const int row = 16 * I + j;
    const float bi = ps.beta[row];
    float mq[4], lk[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int col = 4 * g + r;
      mq[r] = (I > J || col <= j) ? aq[r] : 0.f;        // diagonal kept
      lk[r] = (I > J || col < j) ? bi * ak[r] : 0.f;    // strictly lower
    }
    if constexpr ((PRODUCTS & PROD_MQK) != 0) mqk_sink(row, J, mq);
    if constexpr ((PRODUCTS & PROD_L) != 0) Ar::store4(&L[TL::idx(row, 16 * J + 4 * g)], lk);
  }
}

// Sum of v[0..15] over the 16 lanes of a row group (lanes 16tq + cg), split so
// that lane cg keeps element cg: four halving steps, each lane keeping the
// half its lane bit selects and adding its partner's copy of that half.
__device__ __forceinline__ float reduce_scatter16(const float (&v)[16], int cg) {
  float a[8], b[4], c[2];
  const bool h8 = cg & 8, h4 = cg & 4, h2 = cg & 2, h1 = cg & 1;
#pragma unroll
  for (int x = 0; x < 8; ++x)
    a[x] = (h8 ? v[8 + x] : v[x]) + __shfl_xor(h8 ? v[x] : v[8 + x], 8);
#pragma unroll
  for (int x = 0; x < 4; ++x)
    b[x] = (h4 ? a[4 + x] : a[x]) + __shfl_xor(h4 ? a[x] : a[4 + x], 4);
#pragma unroll
  for (int x = 0; x < 2; ++x)
    c[x] = (h2 ? b[2 + x] : b[x]) + __shfl_xor(h2 ? b[x] : b[2 + x], 2);
  return (h1 ? c[1] : c[0]) + __shfl_xor(h1 ? c[0] : c[1], 1);
}

// LDS writes of this wave become visible to its other lanes (wave-local data)
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// a3 on the diagonal subtiles when the gate has no lower bound and the
// subtile's decay range is too wide for two factors (diag_two_factor fails):
// subtile I = w (this wave's own 16 tokens) from the definition, one position
// pair at a time in fp32, the path that the bound removes ("序列维度（下）",
// section on the 16-token subtiles): for j <= i in the subtile
//   M_qk[i][j] = sum_c q_ic k_jc e^(G_ic - G_jc),
//   L[i][j]    = beta_i sum_c k_ic k_jc e^(G_ic - G_jc)   (j < i only),
// where e^(G_ic - G_jc) <= 1 never overflows.  The wave stages its tokens'
// q, k (as read: bf16 or fp32) and G (fp32) in `stage` (LDS of its own,
// diag_stage_bytes: 8 KB for bf16 inputs, 12 KB for fp32), 64 channels at a
// time.  Lane (tq, cg) takes subtile rows tq, 7 - tq, 8 + tq and 15 - tq (34
// position pairs for every lane) and channels 4cg..4cg+3 of each half; the
// channel sums are then spread over the 16 lanes of the row group, lane cg
// keeping column cg.  M_qk goes to mqk_sink(row, col, value) (zeros above the
// diagonal included), L to the L tile in the operand precision of Ar.
template <class IO> constexpr int diag_stage_bytes() { return 16 * 64 * (4 + 2 * IO::ES); }
template <class IO, class Ar, class MqkSink>
__device__ __forceinline__ void prep_diag_positions(char *stage,
                                                    const typename IO::raw8 (&Rq)[4],
                                                    const typename IO::raw8 (&Rk)[4],
                                                    const float (&G)[4][8], const float *beta,
                                                    typename Ar::E *L, int w, int tq, int cg,
                                                    MqkSink &&mqk_sink) {
  using TL = Tile<typename Ar::E, CH>;
  using SE = typename std::conditional<IO::ES == 2, bf16_t, float>::type;  // staged q, k
  constexpr int HC = 64;  // channels staged at a time
  float *Gs = reinterpret_cast<float *>(stage);               // [16][HC]
  SE *Qs = reinterpret_cast<SE *>(stage + 16 * HC * 4);       // [16][HC]
  SE *Ks = Qs + 16 * HC;                                      // [16][HC]
  auto load4 = [](const SE *x) {
    if constexpr (IO::ES == 2) {
      return Arith<false>::load4(x);
    } else {
      const float4 f = *reinterpret_cast<const float4 *>(x);
      return floatx4{f.x, f.y, f.z, f.w};
    }
  };
  const int c0 = 4 * cg;
#pragma unroll 1
  for (int s = 0; s < 4; ++s) {
    const int row = (s == 0) ? tq : (s == 1) ? 7 - tq : (s == 2) ? 8 + tq : 15 - tq;
    constexpr int NJ_MAX = 16;
    const int nj = 4 * (s + 1);  // rows of slot s are at most 4s + 3
    float m[NJ_MAX], l[NJ_MAX];
#pragma unroll
    for (int jj = 0; jj < NJ_MAX; ++jj) m[jj] = l[jj] = 0.f;
#pragma unroll 1
    for (int hf = 0; hf < 2; ++hf) {
      wave_lds_sync();  // earlier reads of the staging area are done
      if ((cg >> 3) == hf) {
        const int lc = 8 * (cg & 7);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * tq + r;
          *reinterpret_cast<float4 *>(&Gs[i * HC + lc]) = make_float4(G[r][0], G[r][1], G[r][2], G[r][3]);
          *reinterpret_cast<float4 *>(&Gs[i * HC + lc + 4]) = make_float4(G[r][4], G[r][5], G[r][6], G[r][7]);
          if constexpr (IO::ES == 2) {
            *reinterpret_cast<u32x4 *>(&Qs[i * HC + lc]) = Rq[r].a;
            *reinterpret_cast<u32x4 *>(&Ks[i * HC + lc]) = Rk[r].a;
          } else {
            *reinterpret_cast<u32x4 *>(&Qs[i * HC + lc]) = Rq[r].a;
            *reinterpret_cast<u32x4 *>(&Qs[i * HC + lc + 4]) = Rq[r].b;
            *reinterpret_cast<u32x4 *>(&Ks[i * HC + lc]) = Rk[r].a;
            *reinterpret_cast<u32x4 *>(&Ks[i * HC + lc + 4]) = Rk[r].b;
          }
        }
      }
      wave_lds_sync();
      const float4 gi = *reinterpret_cast<const float4 *>(&Gs[row * HC + c0]);
      const floatx4 qi = load4(&Qs[row * HC + c0]);
      const floatx4 ki = load4(&Ks[row * HC + c0]);
      const float giv[4] = {gi.x, gi.y, gi.z, gi.w};
#pragma unroll
      for (int jj = 0; jj < NJ_MAX; ++jj) {
        if (jj < nj) {
          const float4 gj = *reinterpret_cast<const float4 *>(&Gs[jj * HC + c0]);
          const floatx4 kj = load4(&Ks[jj * HC + c0]);
          const float gjv[4] = {gj.x, gj.y, gj.z, gj.w};
          const bool lower = jj <= row;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            // e^(G_i - G_j) in base 2; -inf (factor 0) above the diagonal
            const float x = lower ? giv[c] - gjv[c] : -__builtin_inff();
            const float t = kj[c] * __builtin_amdgcn_exp2f(x);
            m[jj] = fmaf(qi[c], t, m[jj]);
            l[jj] = fmaf(ki[c], t, l[jj]);
          }
        }
      }
    }
    const float mv = reduce_scatter16(m, cg);
    const float lv = reduce_scatter16(l, cg);
    const int i = 16 * w + row;
    mqk_sink(i, 16 * w + cg, mv);
    L[TL::idx(i, 16 * w + cg)] = Ar::cvt(cg < row ? beta[i] * lv : 0.f);
  }
}

// 16x16 tiles in accumulator layout: element r of lane (g, j) is (4g + r, j).
__device__ __forceinline__ floatx4 add_identity(floatx4 x, int g, int j, float s) {
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] += (4 * g + r == j) ? s : 0.f;
  return x;
}

// Inverse of a 16x16 unit lower-triangular I + L with nilpotent L (L^16 = 0):
//   (I + L)^-1 = (I - L)(I + L^2)(I + L^4)(I + L^8).
// A 16x16x16 MFMA takes its A operand row-wise, which is the accumulator layout
// of the transpose, so every power is formed in both orientations:
//   Lt is L^T in accumulator layout (= L in A layout), Ln is L itself.
// Returns T = (I + L)^-1 in accumulator layout.
template <class Ar>
__device__ __forceinline__ floatx4 unit_lower_inverse(floatx4 Ln, floatx4 Lt, int g, int j) {
  const floatx4 z = {0.f, 0.f, 0.f, 0.f};
  floatx4 L2 = Ar::k16(z, Lt, Ln);   // L L        (A = L, B = L)
  floatx4 L2t = Ar::k16(z, Ln, Lt);  // L^T L^T    (A = L^T, B = L^T)
  floatx4 L4 = Ar::k16(z, L2t, L2);
  floatx4 L4t = Ar::k16(z, L2, L2t);
  floatx4 L8t = Ar::k16(z, L4, L4t);
  // R = (I + L^8)(I + L^4)(I + L^2)(I - L), right to left; the factors commute
  floatx4 R = add_identity(-Ln, g, j, 1.f);
  R = R + Ar::k16(z, L2t, R);  // (I + L^2) R
  R = R + Ar::k16(z, L4t, R);  // (I + L^4) R
  R = R + Ar::k16(z, L8t, R);  // (I + L^8) R
  return R;
}

// a4 (i): inverse of the diagonal block w of I + L, stored to Tdg[w] (row-major)
// and returned in accumulator layout.
template <class Ar>
__device__ __forceinline__ floatx4 prep_diag_inverse(const typename Ar::E *L,
                                                     typename Ar::E (*Tdg)[SUB * SUB], int w, int g,
                                                     int j) {
  using TL = Tile<typename Ar::E, CH>;
  floatx4 Ln, Lt;
#pragma unroll
  for (int r = 0; r < 4; ++r) Ln[r] = Ar::tof(L[TL::idx(16 * w + 4 * g + r, 16 * w + j)]);  // L (rows 4g+r, col j)
  Lt = Ar::load4(&L[TL::idx(16 * w + j, 16 * w + 4 * g)]);                               // L^T
  const floatx4 T = unit_lower_inverse<Ar>(Ln, Lt, g, j);
#pragma unroll
  for (int r = 0; r < 4; ++r) Tdg[w][(4 * g + r) * SUB + j] = Ar::cvt(T[r]);
  return T;
}

// Block column J of INV = (I + L)^-1 from the diagonal-block inverses T_II:
//   X_JJ = T_JJ,  X_IJ = -T_II sum_{K=J}^{I-1} L_IK X_KJ  (I > J),
// all tiles in registers (accumulator layout doubles as the 16x16x16 B operand).
// Stores INV Diag(beta) into the 64x64 tile INVb with the token axis permuted.
template <class Ar, int J>
__device__ __forceinline__ void inv_block_column(const typename Ar::E *L,
                                                 const typename Ar::E (*Tdg)[SUB * SUB],
                                                 const float *beta, typename Ar::E *INVb,
                                                 floatx4 Tjj, int g, int j) {
  using TC = Tile<typename Ar::E, CH>;
  using TL = TC;
  floatx4 X[4];
  X[J] = Tjj;
#pragma unroll
  for (int I = J + 1; I < 4; ++I) {
    floatx4 R = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int K = J; K < I; ++K) {
      R = Ar::k16(R, Ar::load4(&L[TL::idx(16 * I + j, 16 * K + 4 * g)]), X[K]);
    }
    const floatx4 t = Ar::load4(&Tdg[I][j * SUB + 4 * g]);  // row j of T_II
    floatx4 Y = {0.f, 0.f, 0.f, 0.f};
    Y = Ar::k16(Y, t, R);
    X[I] = -Y;
  }
  const float bj = beta[16 * J + j];
#pragma unroll
  for (int I = J; I < 4; ++I) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      INVb[TC::idx(16 * I + 4 * g + r, kperm(16 * J + j))] = Ar::cvt(X[I][r] * bj);
  }
}

// a4 (ii): wave w completes block column w (runtime wave index -> template).
template <class Ar>
__device__ __forceinline__ void prep_block_columns(const typename Ar::E *L,
                                                   const typename Ar::E (*Tdg)[SUB * SUB],
                                                   const float *beta, typename Ar::E *INVb,
                                                   floatx4 Tww, int w, int g, int j) {
  switch (w) {
    case 0: inv_block_column<Ar, 0>(L, Tdg, beta, INVb, Tww, g, j); break;
    case 1: inv_block_column<Ar, 1>(L, Tdg, beta, INVb, Tww, g, j); break;
    case 2: inv_block_column<Ar, 2>(L, Tdg, beta, INVb, Tww, g, j); break;
    default: inv_block_column<Ar, 3>(L, Tdg, beta, INVb, Tww, g, j); break;
  }
}

// a5: one chunk of the recurrence for this wave's 16 state columns,
//   U = INV Diag(beta) (V - K_decay S);  O = Q_decay S + M_qk U;
//   S <- Diag(gamma^C) S + K_restore^T U,
// with S in fp32 MFMA accumulators (S[m] holds rows 16m + 4g + r, column j of
// the slice) and V in accumulator layout (Vt[m]: tokens 16m + 4g + r).  The
// operand tiles are the permuted-k LDS tiles the prep stages produce.  O rows
// go through the bounded descriptor ro (tokens past the chunk are dropped) at
// byte offset off_v + token * rowb; write_o = false skips O.
template <class Ar, class IO>
__device__ __forceinline__ void chunk_recurrence(const typename Ar::E *Kd, const typename Ar::E *Qd,
                                                 const typename Ar::E *KrT, const typename Ar::E *Mqk,
                                                 const typename Ar::E *INVb, const float *gamC,
                                                 floatx4 (&S)[8], const floatx4 (&Vt)[4],
                                                 bool write_o, __amdgpu_buffer_rsrc_t ro, int off_v,
                                                 int rowb, int g, int j) {
  using BReg = typename Ar::BReg;
  BReg sb[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) sb[kb] = Ar::breg(S[2 * kb], S[2 * kb + 1]);

  floatx4 U[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    floatx4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) x = Ar::template k32<D>(x, Kd, 16 * m + j, kb, g, sb[kb]);
    U[m] = Vt[m] - x;  // V - K_decay S (Diag(beta) is folded into INV)
  }
  SCHED_FENCE();
  BReg bb[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) bb[kb] = Ar::breg(U[2 * kb], U[2 * kb + 1]);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    floatx4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb <= (m >> 1); ++kb) x = Ar::template k32<CH>(x, INVb, 16 * m + j, kb, g, bb[kb]);
    U[m] = x;
  }
  SCHED_FENCE();
  BReg ub[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) ub[kb] = Ar::breg(U[2 * kb], U[2 * kb + 1]);

  // O = Q_decay S + M_qk U  (off the serial state path)
  if (write_o) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      floatx4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) x = Ar::template k32<D>(x, Qd, 16 * m + j, kb, g, sb[kb]);
#pragma unroll
      for (int kb = 0; kb <= (m >> 1); ++kb) x = Ar::template k32<CH>(x, Mqk, 16 * m + j, kb, g, ub[kb]);
#pragma unroll
      for (int r = 0; r < 4; ++r) IO::st1(ro, x[r], off_v + (16 * m + r) * rowb);
    }
  }
  SCHED_FENCE();
  // S <- Diag(gamma^C) S + K_restore^T U
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const float4 gc = *reinterpret_cast<const float4 *>(&gamC[16 * m + 4 * g]);
    floatx4 x = S[m];
    x[0] *= gc.x; x[1] *= gc.y; x[2] *= gc.z; x[3] *= gc.w;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) x = Ar::template k32<CH>(x, KrT, 16 * m + j, kb, g, ub[kb]);
    S[m] = x;
  }
  SCHED_FENCE();
}

}  // namespace kda
