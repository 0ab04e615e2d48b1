// kda_prefill.hip -- chunkwise KDA prefill for gfx950.
//
// One workgroup (4 waves) runs the serial chunk chain of one (item, head,
// 64-column slice of the state).  An item is a document of the packed sequence
// (mode 0), or a fixed token range that may contain document starts: a segment
// re-run from its scanned entry state (mode 1) or a segment pair (M, S~) built
// from a zero state (mode 2).  Per chunk of C = 64 tokens the workgroup does
//
//   prep (token-parallel, all waves; the "chunk prep" of the pages)
//     a1  gate g = g_min*sigmoid(exp(A_h) z) and the in-chunk inclusive
//         cumulative log-decay G ("序列维度（下）", eq. (3), eq. (5), section
//         "数值问题"), in base-2 units;
//     a2  decay factors Q_decay = e^G q, K_decay = e^G k, K_restore =
//         e^(G_C - G) k and the 16-token subtile operands referenced to the
//         first token s of the query subtile: e^(G_i - G_s) <= 1 on the query
//         side, e^(G_s - G_j) < e^75 on the key side (g > g_min = -5 keeps it
//         inside the bf16 range, section "K3 的改动：下界衰减");
//     a3  L = StrictTril(Diag(beta) K_decay K_inv^T) and M_qk =
//         Tril(Q_decay K_inv^T) (diagonal kept) per 16x16 subtile pair on MFMA
//         (SemiAnalysis page, section "FlashKDA 算法");
//     a4  the UT transform INV = (I + L)^-1 ("序列维度（下）", section "UT 变换"):
//         each 16x16 diagonal block by repeated squaring,
//         (I + L)^-1 = (I - L)(I + L^2)(I + L^4)(I + L^8), then each wave
//         completes one block column X_IJ = -T_II sum_K L_IK X_KJ; INV Diag(beta)
//         is kept for the recurrence;
//   recurrence (serial over chunks; each wave owns 16 state columns)
//     a5  U = INV Diag(beta) (V - K_decay S);  O = Q_decay S + M_qk U;
//         S <- Diag(gamma^C) S + K_restore^T U,
//         with S held in fp32 MFMA accumulators for the whole chain.
//
// Arithmetic: bf16 MFMA operands with fp32 accumulation (F32C = false) or an
// fp32-MFMA verification build (F32C = true) from the same source.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int FWD_THREADS = 256;
constexpr float LOG2E = 1.4426950408889634f;

// Keep the instruction scheduler from moving work across chunk phases.
#define SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// ---------------------------------------------------------------------------
// LDS.  Subtile operands (phase 1: natural channel order) and recurrence
// operands (phase 2: k axis permuted, see kperm).  With bf16 operands both fit
// at once and phase 2 is written as soon as it is computed; the fp32
// verification build overlays them and keeps phase 2 in registers until
// phase 1 has been consumed.  Every operand tile is XOR-swizzled (Tile<>).
// ---------------------------------------------------------------------------
template <typename E> struct P1 {
  E Qh[CH * D];  // q_i e^(G_i - G_s(i))
  E Kh[CH * D];  // k_i e^(G_i - G_s(i))
  E Ki[CH * D];  // k_j e^(G_s(j) - G_j)
};
template <typename E> struct P2 {
  E Kd[CH * D];   // K_decay, channel axis permuted
  E Qd[CH * D];   // Q_decay, channel axis permuted
  E KrT[D * CH];  // K_restore^T, token axis permuted
};
template <typename E, bool ALIAS> struct POps;
template <typename E> struct POps<E, true> { union { P1<E> p1; P2<E> p2; }; };
template <typename E> struct POps<E, false> { P1<E> p1; P2<E> p2; };

template <typename E, bool ALIAS>
struct __align__(16) FwdSmem {
  POps<E, ALIAS> A;
  E Mqk[CH * CH];    // token (column) axis permuted; upper 16x16 blocks stay 0
  E INVb[CH * CH];   // INV Diag(beta); token axis permuted; upper blocks stay 0
  float L[CH * CH];  // strict lower part used
  E Tdg[4][SUB * SUB];  // inverses of the diagonal 16x16 blocks of I + L
  float gamC[D];        // gamma^C = e^(G_C)
  float GC2[D];         // G_C (base 2)
  float Gref[4][D];     // G (base 2) at the first token of each subtile
  float F[6][D];        // e^(Gref[I] - Gref[J]) for I > J
  float beta[CH];
  float wtot[4][D];     // per-wave cumulative-sum totals
};

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

// document offsets; cu == nullptr means one document [0, T)
__device__ __forceinline__ int64_t cu_at(const FwdParams &p, int i) {
  return p.cu ? (int64_t)p.cu[i] : (i == 0 ? (int64_t)0 : p.T);
}
// largest d in [0, N-1] with cu[d] <= pos (skips empty documents starting at pos)
__device__ __forceinline__ int doc_of(const int32_t *cu, int N, int64_t pos) {
  if (!cu) return 0;
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= pos) lo = mid; else hi = mid - 1;
  }
  return uni(lo);
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

// Block column J of INV = (I + L)^-1 from the diagonal-block inverses T_II:
//   X_JJ = T_JJ,  X_IJ = -T_II sum_{K=J}^{I-1} L_IK X_KJ  (I > J),
// all tiles in registers (accumulator layout doubles as the 16x16x16 B operand).
// Stores INV Diag(beta) into INVb with the token axis permuted.
template <class Ar, int J, class Smem>
__device__ __forceinline__ void inv_block_column(Smem &sm, floatx4 Tjj, int g, int j) {
  using E = typename Ar::E;
  using TC = Tile<E, CH>;
  using TL = Tile<float, CH>;
  floatx4 X[4];
  X[J] = Tjj;
#pragma unroll
  for (int I = J + 1; I < 4; ++I) {
    floatx4 R = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int K = J; K < I; ++K) {
      const float4 l4 = *reinterpret_cast<const float4 *>(&sm.L[TL::idx(16 * I + j, 16 * K + 4 * g)]);
      R = Ar::k16(R, floatx4{l4.x, l4.y, l4.z, l4.w}, X[K]);
    }
    const floatx4 t = Ar::load4(&sm.Tdg[I][j * SUB + 4 * g]);  // row j of T_II
    floatx4 Y = {0.f, 0.f, 0.f, 0.f};
    Y = Ar::k16(Y, t, R);
    X[I] = -Y;
  }
  const float bj = sm.beta[16 * J + j];
#pragma unroll
  for (int I = J; I < 4; ++I) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      sm.INVb[TC::idx(16 * I + 4 * g + r, kperm(16 * J + j))] = Ar::cvt(X[I][r] * bj);
  }
}

// Recurrence operands of one token (8 channels) into LDS: K_decay and Q_decay
// rows, channels 8cg..8cg+7 = two groups of 4 consecutive permuted positions.
template <class Ar, class Smem>
__device__ __forceinline__ void write_phase2_row(Smem &sm, const float (&Kdec)[8],
                                                 const float (&Qdec)[8], int i, int cg) {
  using TD = Tile<typename Ar::E, D>;
  Ar::store4(&sm.A.p2.Kd[TD::idx(i, kperm(8 * cg))], &Kdec[0]);
  Ar::store4(&sm.A.p2.Kd[TD::idx(i, kperm(8 * cg + 4))], &Kdec[4]);
  Ar::store4(&sm.A.p2.Qd[TD::idx(i, kperm(8 * cg))], &Qdec[0]);
  Ar::store4(&sm.A.p2.Qd[TD::idx(i, kperm(8 * cg + 4))], &Qdec[4]);
}
// K_restore^T for this thread's 4 tokens (consecutive permuted positions) x 8 channels.
template <class Ar, class Smem>
__device__ __forceinline__ void write_phase2_krt(Smem &sm, const float (&Kres)[4][8], int w,
                                                 int tq, int cg) {
  using TC = Tile<typename Ar::E, CH>;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float x[4] = {Kres[0][c], Kres[1][c], Kres[2][c], Kres[3][c]};
    Ar::store4(&sm.A.p2.KrT[TC::idx(8 * cg + c, kperm(16 * w + 4 * tq))], x);
  }
}

template <typename Tin, bool F32C>
__global__ void __launch_bounds__(FWD_THREADS, 1) kda_fwd_kernel(FwdParams p) {
  using Ar = Arith<F32C>;
  using E = typename Ar::E;
  using BReg = typename Ar::BReg;
  using IO = bufio<Tin>;
  using TD = Tile<E, D>;    // 64 x 128 operand tiles
  using TC = Tile<E, CH>;   // 128 x 64 and 64 x 64 operand tiles
  using TL = Tile<float, CH>;
  constexpr int NT = 1;     // 16 state columns per wave
  constexpr bool ALIAS = F32C;  // fp32 operands: overlay phase 1 and phase 2 in LDS
  constexpr int ES = IO::ES;
  __shared__ FwdSmem<E, ALIAS> sm;

  // ---- which (item, head, slice) this workgroup runs; slices of one
  //      (item, head) share an XCD (blockIdx % 8) so they share L2 ----------
  const int units = p.n_items * p.H;
  const int xlo = blockIdx.x & 7;
  const int rest = blockIdx.x >> 3;
  const int split = rest % p.nsplit;
  const int unit = (rest / p.nsplit) * 8 + xlo;
  if (unit >= units) return;
  const int item = unit / p.H;
  const int h = unit % p.H;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;     // wave; also the subtile it owns in prep
  const int g = lane >> 4;    // MFMA lane group
  const int j = lane & 15;    // MFMA lane column
  const int tq = lane >> 4;   // prep: 4-token group inside the subtile
  const int cg = lane & 15;   // prep: 8-channel group
  const int colW = split * (64 * NT) + w * (16 * NT);  // first state column of this wave
  const int H = p.H;

  int64_t a, b;
  int doc;
  // mode 2: slices 0,1 carry S~ (value columns), slices 2,3 carry M (identity start, v = 0)
  const bool m_cols = (p.mode == 2) && (colW >= D);
  const float *init_src = nullptr;  // initial state (row-major D x D), nullptr = 0 / identity
  if (p.mode == 0) {
    a = cu_at(p, item);
    b = cu_at(p, item + 1);
    if (a == b) return;  // empty documents are handled by kda_copy_empty_kernel
    doc = item;
    if (p.item_init) init_src = p.item_init + ((int64_t)doc * H + h) * (D * D);
  } else {
    a = (int64_t)item * p.seg_len;
    b = min(p.T, a + p.seg_len);
    if (p.mode == 1) {
      doc = doc_of(p.cu, p.N, a);
      init_src = p.item_init + ((int64_t)item * H + h) * (D * D);
    } else {
      // The pair maps the state at the segment start to the state at its end.
      // If a document starts strictly inside, the end state does not depend on
      // the entry state (M = 0) and S~ runs from that document's own state.
      doc = doc_of(p.cu, p.N, b - 1);
      const int64_t ds = uni64(cu_at(p, doc));
      if (ds > a) {
        if (m_cols) {
          float *dst = p.final_state + ((int64_t)item * H + h) * (D * 2 * D);
          for (int x = tid; x < D * 64 * NT; x += FWD_THREADS)
            dst[(x / (64 * NT)) * (2 * D) + split * (64 * NT) + x % (64 * NT)] = 0.f;
          return;
        }
        a = ds;
        if (p.doc_init) init_src = p.doc_init + ((int64_t)doc * H + h) * (D * D);
      }
    }
  }
  a = uni64(a);
  b = uni64(b);
  if (init_src) init_src = uniptr(init_src);

  const Tin *q = (const Tin *)p.q;
  const Tin *k = (const Tin *)p.k;
  const Tin *v = (const Tin *)p.v;
  const Tin *z = (const Tin *)p.z;
  const Tin *bt = (const Tin *)p.beta;
  Tin *o = (Tin *)p.o;
  const float c1 = -__expf(p.A_log ? p.A_log[h] : 0.0f) * LOG2E;  // gate: exp2(c1 z)
  const float gmin2 = p.g_min * LOG2E;
  const int rowb = H * D * ES;  // bytes between consecutive tokens of one head

  // M_qk and INV Diag(beta) keep zero upper 16x16 blocks for the whole chain.
  for (int x = tid; x < CH * CH; x += FWD_THREADS) {
    sm.Mqk[x] = Ar::cvt(0.f);
    sm.INVb[x] = Ar::cvt(0.f);
  }

  // ---- initial state, in accumulator layout: S[m][n] holds rows 16m+4g+r,
  //      column colW + 16n + j --------------------------------------------
  floatx4 S[8][NT];
  if (m_cols) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S[m][n][r] = (16 * m + 4 * g + r == colW + 16 * n + j - D) ? 1.f : 0.f;
  } else if (init_src) {
    state_load(S, init_src, D, colW, g, j);
  } else {
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n) S[m][n] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  int64_t doc_end = (p.mode == 2) ? b : uni64(cu_at(p, doc + 1));

  // Per-lane byte offsets (loop-invariant) into a chunk's rows of q, k, z
  // (token 16w + 4tq + r, channels 8cg..) and of v / o (token 16m + 4g + r,
  // column colW + j).  Chunk bases are wave-uniform; descriptors are bounded at
  // the chunk's last valid token, so tail rows read 0 and are not written.
  const int off_qkz = ((16 * w + 4 * tq) * H * D + 8 * cg) * ES;
  const int off_v = (4 * g * H * D + colW + j) * ES;
  const int vcol_ok = !m_cols;

  typename IO::raw8 Rq[4], Rk[4], Rz[4];
  typename IO::raw1 Rv[4][4], Rb;
  auto fetch = [&](int64_t c0, int n) {
    const int bytes = ((n - 1) * H + 1) * D * ES;
    const int64_t e0 = (c0 * H + h) * D;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + e0, bytes);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + e0, bytes);
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(z + e0, bytes);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      Rq[r] = IO::ld8(rq, off_qkz + r * rowb);
      Rk[r] = IO::ld8(rk, off_qkz + r * rowb);
      Rz[r] = IO::ld8(rz, off_qkz + r * rowb);
    }
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + e0, vcol_ok ? bytes : 0);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) Rv[m][r] = IO::ld1(rv, off_v + (16 * m + r) * rowb);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(bt + (c0 * H + h), ((n - 1) * H + 1) * ES);
    Rb = IO::ld1(rb, (tid & 63) * H * ES);
  };

  int64_t pos = a;
  int len_next = (int)min((int64_t)CH, min(b, doc_end) - a);
  if (len_next > 0) fetch(a, len_next);
  while (pos < b) {
    const int64_t cs = pos;
    const int len = len_next;
    if (len <= 0) break;  // only if device and host offsets disagree; never loop forever

    // ================= prep (a1-a4) =================
    // a1: gate of z for tokens 16w + 4tq + r, channels 8cg..8cg+7 (base 2)
    float G[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float gm = (16 * w + 4 * tq + r < len) ? gmin2 : 0.f;  // padding rows: no decay
      float zz[8];
      IO::cvt8(Rz[r], zz);
#pragma unroll
      for (int c = 0; c < 8; ++c) G[r][c] = kda_gate2(zz[c], c1, gm);
    }
    if (tid < CH) sm.beta[tid] = IO::cvt1(Rb);
    // V in accumulator layout (tokens 16m + 4g + r, this wave's columns)
    floatx4 Vt[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) Vt[m][r] = IO::cvt1(Rv[m][r]);
    // where the next chunk starts (chunks restart at document starts)
    int64_t npos, nlen;
    {
      npos = cs + len;
      int64_t nend = doc_end;
      if (p.mode != 2 && npos == doc_end && npos < b) nend = uni64(cu_at(p, doc_of(p.cu, p.N, npos) + 1));
      nlen = (npos < b) ? min((int64_t)CH, min(b, nend) - npos) : 0;
    }

    // inclusive cumulative sum over the chunk: in-lane over r, across the
    // 4 token groups of the wave (lanes 16 apart), then across waves.
    {
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
        const float4 lo = make_float4(G[3][0], G[3][1], G[3][2], G[3][3]);
        const float4 hi = make_float4(G[3][4], G[3][5], G[3][6], G[3][7]);
        *reinterpret_cast<float4 *>(&sm.wtot[w][8 * cg]) = lo;
        *reinterpret_cast<float4 *>(&sm.wtot[w][8 * cg + 4]) = hi;
      }
    }
    __syncthreads();  // B1
    SCHED_FENCE();
    {
      float off[8];
      const float4 t0a = *reinterpret_cast<const float4 *>(&sm.wtot[0][8 * cg]);
      const float4 t0b = *reinterpret_cast<const float4 *>(&sm.wtot[0][8 * cg + 4]);
      const float4 t1a = *reinterpret_cast<const float4 *>(&sm.wtot[1][8 * cg]);
      const float4 t1b = *reinterpret_cast<const float4 *>(&sm.wtot[1][8 * cg + 4]);
      const float4 t2a = *reinterpret_cast<const float4 *>(&sm.wtot[2][8 * cg]);
      const float4 t2b = *reinterpret_cast<const float4 *>(&sm.wtot[2][8 * cg + 4]);
      const float t0[8] = {t0a.x, t0a.y, t0a.z, t0a.w, t0b.x, t0b.y, t0b.z, t0b.w};
      const float t1[8] = {t1a.x, t1a.y, t1a.z, t1a.w, t1b.x, t1b.y, t1b.z, t1b.w};
      const float t2[8] = {t2a.x, t2a.y, t2a.z, t2a.w, t2b.x, t2b.y, t2b.z, t2b.w};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        off[c] = (w > 0 ? t0[c] : 0.f) + (w > 1 ? t1[c] : 0.f) + (w > 2 ? t2[c] : 0.f);
#pragma unroll
        for (int r = 0; r < 4; ++r) G[r][c] += off[c];
      }
    }
    if (tq == 0) {
      *reinterpret_cast<float4 *>(&sm.Gref[w][8 * cg]) = make_float4(G[0][0], G[0][1], G[0][2], G[0][3]);
      *reinterpret_cast<float4 *>(&sm.Gref[w][8 * cg + 4]) = make_float4(G[0][4], G[0][5], G[0][6], G[0][7]);
    }
    if (w == 3 && tq == 3) {
      *reinterpret_cast<float4 *>(&sm.GC2[8 * cg]) = make_float4(G[3][0], G[3][1], G[3][2], G[3][3]);
      *reinterpret_cast<float4 *>(&sm.GC2[8 * cg + 4]) = make_float4(G[3][4], G[3][5], G[3][6], G[3][7]);
    }
    __syncthreads();  // B2
    SCHED_FENCE();

    // a2: subtile operands (phase 1) and recurrence operands (phase 2)
    float Kdec[4][8], Qdec[4][8], Kres[4][8];
    {
      float Pj[8], Rj[8], gref[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        gref[c] = sm.Gref[w][8 * cg + c];
        Pj[c] = __builtin_amdgcn_exp2f(gref[c]);                       // e^(G_s)
        Rj[c] = __builtin_amdgcn_exp2f(sm.GC2[8 * cg + c] - gref[c]);  // e^(G_C - G_s) <= 1
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * w + 4 * tq + r;
        float qv[8], kv[8], qh[8], kh[8], ki[8];
        IO::cvt8(Rq[r], qv);
        IO::cvt8(Rk[r], kv);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float e1 = __builtin_amdgcn_exp2f(G[r][c] - gref[c]);  // <= 1
          const float e2 = __builtin_amdgcn_rcpf(e1);                   // < e^75
          qh[c] = qv[c] * e1;
          kh[c] = kv[c] * e1;
          ki[c] = kv[c] * e2;
          Qdec[r][c] = qh[c] * Pj[c];
          Kdec[r][c] = kh[c] * Pj[c];
          Kres[r][c] = ki[c] * Rj[c];
        }
        Ar::store4(&sm.A.p1.Qh[TD::idx(i, 8 * cg)], qh);
        Ar::store4(&sm.A.p1.Qh[TD::idx(i, 8 * cg + 4)], qh + 4);
        Ar::store4(&sm.A.p1.Kh[TD::idx(i, 8 * cg)], kh);
        Ar::store4(&sm.A.p1.Kh[TD::idx(i, 8 * cg + 4)], kh + 4);
        Ar::store4(&sm.A.p1.Ki[TD::idx(i, 8 * cg)], ki);
        Ar::store4(&sm.A.p1.Ki[TD::idx(i, 8 * cg + 4)], ki + 4);
        if constexpr (!ALIAS) write_phase2_row<Ar>(sm, Kdec[r], Qdec[r], i, cg);
        SCHED_FENCE();
      }
      if constexpr (!ALIAS) write_phase2_krt<Ar>(sm, Kres, w, tq, cg);
      // F[pair][c] = e^(Gref[I][c] - Gref[J][c]), pairs (1,0),(2,0),(2,1),(3,0),(3,1),(3,2)
      for (int x = tid; x < 6 * D; x += FWD_THREADS) {
        const int pi = x / D, c = x % D;
        const int I = (pi == 0) ? 1 : (pi < 3 ? 2 : 3);
        const int J = (pi == 0) ? 0 : (pi < 3 ? pi - 1 : pi - 3);
        sm.F[pi][c] = __builtin_amdgcn_exp2f(sm.Gref[I][c] - sm.Gref[J][c]);
      }
      if (tid < D) sm.gamC[tid] = __builtin_amdgcn_exp2f(sm.GC2[tid]);
    }
    SCHED_FENCE();
    if (nlen > 0) fetch(npos, (int)nlen);  // next chunk's inputs stream in behind this one
    len_next = (int)nlen;
    __syncthreads();  // B3
    SCHED_FENCE();

    // a3: A_qk and A_kk per subtile pair (I >= J); wave w takes pairs w, w+4, w+8.
    // Products are formed transposed, (K_inv_J)(Q_I)^T, so lane (g, i) ends up
    // with row i of the pair's tile at columns 4g..4g+3 and writes them at once.
    for (int pidx = w; pidx < 10; pidx += 4) {
      const int I = (pidx == 0) ? 0 : (pidx < 3 ? 1 : (pidx < 6 ? 2 : 3));
      const int J = pidx - I * (I + 1) / 2;
      floatx4 aq = {0.f, 0.f, 0.f, 0.f}, ak = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        BReg kin;  // key side of subtile J, referenced to the first token of subtile I
        if (I == J) {
          kin = Ar::template breg_lds<D>(sm.A.p1.Ki, 16 * J + j, kb, g);
        } else {
          const int fp = I * (I - 1) / 2 + J;
          kin = Ar::template breg_lds_scaled<D>(sm.A.p1.Ki, 16 * J + j, kb, g, sm.F[fp]);
        }
        aq = Ar::template k32_regA<D>(aq, kin, sm.A.p1.Qh, 16 * I + j, kb, g);
        ak = Ar::template k32_regA<D>(ak, kin, sm.A.p1.Kh, 16 * I + j, kb, g);
      }
      // lane (g, j): element r is (row j of subtile I, column 4g + r of subtile J)
      const int row = 16 * I + j;
      const float bi = sm.beta[row];
      float mq[4], lk[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = 4 * g + r;
        mq[r] = (I > J || col <= j) ? aq[r] : 0.f;        // diagonal kept
        lk[r] = (I > J || col < j) ? bi * ak[r] : 0.f;    // strictly lower
      }
      Ar::store4(&sm.Mqk[TC::idx(row, kperm(16 * J + 4 * g))], mq);
      *reinterpret_cast<float4 *>(&sm.L[TL::idx(row, 16 * J + 4 * g)]) = make_float4(lk[0], lk[1], lk[2], lk[3]);
    }
    __syncthreads();  // B4: phase-1 operands dead, L complete
    SCHED_FENCE();

    if constexpr (ALIAS) {  // phase 2 operands into the LDS region phase 1 occupied
#pragma unroll
      for (int r = 0; r < 4; ++r) write_phase2_row<Ar>(sm, Kdec[r], Qdec[r], 16 * w + 4 * tq + r, cg);
      write_phase2_krt<Ar>(sm, Kres, w, tq, cg);
    }
    // a4 (i): inverse of the diagonal block w of I + L
    floatx4 Tww;
    {
      floatx4 Ln, Lt;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Ln[r] = sm.L[TL::idx(16 * w + 4 * g + r, 16 * w + j)];  // L (rows 4g+r, col j)
        Lt[r] = sm.L[TL::idx(16 * w + j, 16 * w + 4 * g + r)];  // L^T
      }
      Tww = unit_lower_inverse<Ar>(Ln, Lt, g, j);
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.Tdg[w][(4 * g + r) * SUB + j] = Ar::cvt(Tww[r]);
    }
    __syncthreads();  // B5
    SCHED_FENCE();
    // a4 (ii): block column J = w of INV: X_IJ = -T_II sum_{K=J}^{I-1} L_IK X_KJ
    switch (w) {
      case 0: inv_block_column<Ar, 0>(sm, Tww, g, j); break;
      case 1: inv_block_column<Ar, 1>(sm, Tww, g, j); break;
      case 2: inv_block_column<Ar, 2>(sm, Tww, g, j); break;
      default: inv_block_column<Ar, 3>(sm, Tww, g, j); break;
    }
    __syncthreads();  // B6
    SCHED_FENCE();

    // ================= recurrence (a5) =================
    BReg sb[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sb[kb] = Ar::breg(S[2 * kb][0], S[2 * kb + 1][0]);

    floatx4 U[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      floatx4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) x = Ar::template k32<D>(x, sm.A.p2.Kd, 16 * m + j, kb, g, sb[kb]);
      U[m] = Vt[m] - x;  // B' = V - K_decay S (Diag(beta) is folded into INV)
    }
    SCHED_FENCE();
    BReg bb[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) bb[kb] = Ar::breg(U[2 * kb], U[2 * kb + 1]);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      floatx4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb <= (m >> 1); ++kb) x = Ar::template k32<CH>(x, sm.INVb, 16 * m + j, kb, g, bb[kb]);
      U[m] = x;
    }
    SCHED_FENCE();
    BReg ub[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) ub[kb] = Ar::breg(U[2 * kb], U[2 * kb + 1]);

    // O = Q_decay S + M_qk U  (off the serial state path)
    if (p.mode != 2) {
      const __amdgpu_buffer_rsrc_t ro = make_rsrc(o + (cs * H + h) * D, ((len - 1) * H + 1) * D * ES);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        floatx4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) x = Ar::template k32<D>(x, sm.A.p2.Qd, 16 * m + j, kb, g, sb[kb]);
#pragma unroll
        for (int kb = 0; kb <= (m >> 1); ++kb) x = Ar::template k32<CH>(x, sm.Mqk, 16 * m + j, kb, g, ub[kb]);
#pragma unroll
        for (int r = 0; r < 4; ++r) IO::st1(ro, x[r], off_v + (16 * m + r) * rowb);
      }
    }
    SCHED_FENCE();
    // S <- Diag(gamma^C) S + K_restore^T U
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float4 gc = *reinterpret_cast<const float4 *>(&sm.gamC[16 * m + 4 * g]);
      floatx4 x = S[m][0];
      x[0] *= gc.x; x[1] *= gc.y; x[2] *= gc.z; x[3] *= gc.w;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) x = Ar::template k32<CH>(x, sm.A.p2.KrT, 16 * m + j, kb, g, ub[kb]);
      S[m][0] = x;
    }

    SCHED_FENCE();
    pos += len;
    if (p.mode == 2) {
      if (pos == b)  // emit the pair [S~ | M] for this segment
        state_store(S, uniptr(p.final_state + ((int64_t)item * H + h) * (D * 2 * D)), 2 * D, colW, g, j);
    } else if (pos == doc_end) {
      // document boundary: emit its final state, then reset for the next document
      if (p.final_state) state_store(S, uniptr(p.final_state + ((int64_t)doc * H + h) * (D * D)), D, colW, g, j);
      if (pos < b) {
        doc = doc_of(p.cu, p.N, pos);
        doc_end = uni64(cu_at(p, doc + 1));
        if (p.doc_init) {
          state_load(S, uniptr(p.doc_init + ((int64_t)doc * H + h) * (D * D)), D, colW, g, j);
        } else {
#pragma unroll
          for (int m = 0; m < 8; ++m) S[m][0] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    // The next chunk writes beta, wtot, Gref, GC2 before touching anything the
    // recurrence reads, except with overlaid operands (ALIAS), where phase 1
    // of the next chunk overwrites phase 2 of this one.
    if constexpr (ALIAS) __syncthreads();  // B7
  }
}

// final_state[d] = initial_state[d] (or 0) for empty documents
__global__ void kda_copy_empty_kernel(const int32_t *cu, int64_t T, const float *init, float *fin,
                                      int H) {
  const int d = blockIdx.x / H, h = blockIdx.x % H;
  const int64_t len = cu ? (int64_t)cu[d + 1] - cu[d] : T;
  if (len != 0) return;
  const int64_t base = ((int64_t)d * H + h) * (D * D);
  for (int x = threadIdx.x; x < D * D; x += blockDim.x) fin[base + x] = init ? init[base + x] : 0.f;
}

template <typename Tin, bool F32C>
static hipError_t launch_fwd_t(const FwdParams &p, hipStream_t stream) {
  const int units = p.n_items * p.H;
  const int groups = (units + 7) / 8;
  const dim3 grid((unsigned)(groups * 8 * p.nsplit));
  hipLaunchKernelGGL((kda_fwd_kernel<Tin, F32C>), grid, dim3(FWD_THREADS), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_fwd(FwdParams p, bool bf16_in, bool f32_compute, hipStream_t stream) {
  // slices of 64 state columns per (item, head), 16 per wave: two for the
  // 128 value columns, four for the [S~ | M] pair columns
  p.nsplit = (p.mode == 2) ? 4 : 2;
  if (bf16_in)
    return f32_compute ? launch_fwd_t<bf16_t, true>(p, stream)
                       : launch_fwd_t<bf16_t, false>(p, stream);
  return f32_compute ? launch_fwd_t<float, true>(p, stream)
                     : launch_fwd_t<float, false>(p, stream);
}

hipError_t launch_copy_empty(const int32_t *cu, int64_t T, const float *init, float *fin, int N,
                             int H, hipStream_t stream) {
  hipLaunchKernelGGL(kda_copy_empty_kernel, dim3((unsigned)(N * H)), dim3(256), 0, stream, cu, T,
                     init, fin, H);
  return hipGetLastError();
}

}  // namespace kda
