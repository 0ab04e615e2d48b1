// kda_prefill.hip -- chunkwise KDA prefill for gfx950.
//
// One workgroup (4 waves) runs the serial chunk chain of one (item, head,
// d_v-slice).  An item is either a document of the packed sequence or, for the
// segment scan, a fixed token range that may contain document starts.  Per
// chunk of C = 64 tokens the workgroup
//
//   prep  (token-parallel, all 4 waves; the "chunk prep" of the pages)
//     a1  gate g = g_min*sigmoid(exp(A_h) z) and the in-chunk inclusive
//         cumulative log-decay G ("序列维度（下）", eq. (3), eq. (5), section
//         "数值问题");
//     a2  decay factors Q_decay = e^G q, K_decay = e^G k,
//         K_restore = e^(G_C - G) k, and the 16-token subtile operands
//         referenced to the first token s of the query subtile
//         (e^(G_i - G_s) on the query side, e^(G_s - G_j) on the key side);
//         because g > g_min = -5 the key-side factor stays below e^75 and fits
//         bf16 (section "K3 的改动：下界衰减");
//     a3  L = StrictTril(Diag(beta) K_decay K_inv^T) and
//         M_qk = Tril(Q_decay K_inv^T) (diagonal kept), per 16x16 subtile pair
//         on MFMA (SemiAnalysis page, section "FlashKDA 算法");
//     a4  the UT transform INV = (I + L)^-1 ("序列维度（下）", section "UT 变换"):
//         16x16 diagonal blocks by forward substitution in fp32, then each
//         wave completes one block column with 16x16x16 MFMA steps held in
//         registers; INV Diag(beta) is stored for the recurrence;
//   recurrence (serial over chunks; each wave owns 16*NT state columns)
//     a5  U = INV Diag(beta) (V - K_decay S);  O = Q_decay S + M_qk U;
//         S <- Diag(gamma^C) S + K_restore^T U,
//         with S kept in fp32 MFMA accumulators for the whole chain.
//
// Arithmetic: bf16 MFMA operands with fp32 accumulation (F32C = false) or an
// fp32-MFMA verification build (F32C = true) from the same source.
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int FWD_THREADS = 256;

// Keep the instruction scheduler from moving work across chunk phases: without
// it the LDS operand reads of every MFMA of a phase get hoisted together and the
// kernel runs out of registers.
#define SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// Subtile operands (phase 1: natural channel order) and recurrence operands
// (phase 2: k axis permuted, see kperm).  With bf16 operands both fit in LDS at
// once and phase 2 is written as soon as it is computed; the fp32 verification
// build overlays them and keeps phase 2 in registers until phase 1 is consumed.
template <typename E> struct P1 {
  E Qh[CH][D];  // q_i e^(G_i - G_s(i))
  E Kh[CH][D];  // k_i e^(G_i - G_s(i))
  E Ki[CH][D];  // k_j e^(G_s(j) - G_j)
};
template <typename E> struct P2 {
  E Kd[CH][D];   // K_decay, channel axis permuted
  E Qd[CH][D];   // Q_decay, channel axis permuted
  E KrT[D][CH];  // K_restore^T, token axis permuted
};
template <typename E, bool ALIAS> struct POps;
template <typename E> struct POps<E, true> { union { P1<E> p1; P2<E> p2; }; };
template <typename E> struct POps<E, false> { P1<E> p1; P2<E> p2; };

template <typename E, bool ALIAS>
struct __align__(16) FwdSmem {
  POps<E, ALIAS> A;
  E Mqk[CH][CH];    // token (column) axis permuted; upper 16x16 blocks stay 0
  E INVb[CH][CH];   // INV Diag(beta); token axis permuted; upper blocks stay 0
  float L[CH][CH];  // strict lower part used
  E Tdg[4][SUB][SUB];  // inverses of the diagonal 16x16 blocks of I + L
  float gamC[D];       // gamma^C = e^(G_C)
  float Gref[4][D];    // G at the first token of each subtile
  float F[6][D];       // e^(Gref[I] - Gref[J]) for I > J
  float beta[CH];
  float wtot[4][D];    // per-wave cumulative-sum totals
};

// ---------------------------------------------------------------------------
// MFMA operand plumbing for the two arithmetic modes.
// ---------------------------------------------------------------------------
template <bool F32C> struct Arith;

template <> struct Arith<false> {  // bf16 operands, fp32 accumulate
  using E = bf16_t;
  struct BReg { bf16x8 v; };
  static __device__ __forceinline__ E cvt(float x) { return f32_to_bf16(x); }
  static __device__ __forceinline__ float tof(E x) { return bf16_to_f32(x); }
  static __device__ __forceinline__ BReg breg(floatx4 t0, floatx4 t1) {
    BReg b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      b.v[e] = (__bf16)t0[e];
      b.v[4 + e] = (__bf16)t1[e];
    }
    return b;
  }
  // acc += A[row pa][8g..8g+8) . B  (B from registers)
  static __device__ __forceinline__ floatx4 k32(floatx4 acc, const E *pa, int g, const BReg &b) {
    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(pa + 8 * g);
    return mfma_bf16_k32(a, b.v, acc);
  }
  // B operand read from an LDS row (natural order), optionally scaled per k
  static __device__ __forceinline__ BReg breg_lds(const E *pb, int g) {
    BReg b;
    b.v = *reinterpret_cast<const bf16x8 *>(pb + 8 * g);
    return b;
  }
  static __device__ __forceinline__ BReg breg_lds_scaled(const E *pb, int g, const float *sc) {
    const bf16x8 raw = *reinterpret_cast<const bf16x8 *>(pb + 8 * g);
    const float4 s0 = *reinterpret_cast<const float4 *>(sc + 8 * g);
    const float4 s1 = *reinterpret_cast<const float4 *>(sc + 8 * g + 4);
    const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    BReg b;
#pragma unroll
    for (int e = 0; e < 8; ++e) b.v[e] = (__bf16)((float)raw[e] * s[e]);
    return b;
  }
  // 16x16x16 step: acc += A[row pa][4g..4g+4) (fp32 or E in LDS) . t (acc layout)
  static __device__ __forceinline__ floatx4 k16_f32a(floatx4 acc, const float *pa, int g,
                                                     floatx4 t) {
    const float4 a4 = *reinterpret_cast<const float4 *>(pa + 4 * g);
    bf16x4 a, b;
    a[0] = (__bf16)a4.x; a[1] = (__bf16)a4.y; a[2] = (__bf16)a4.z; a[3] = (__bf16)a4.w;
#pragma unroll
    for (int e = 0; e < 4; ++e) b[e] = (__bf16)t[e];
    return mfma_bf16_k16(a, b, acc);
  }
  static __device__ __forceinline__ floatx4 k16_ea(floatx4 acc, const E *pa, int g, floatx4 t) {
    const bf16x4 a = *reinterpret_cast<const bf16x4 *>(pa + 4 * g);
    bf16x4 b;
#pragma unroll
    for (int e = 0; e < 4; ++e) b[e] = (__bf16)t[e];
    return mfma_bf16_k16(a, b, acc);
  }
  static __device__ __forceinline__ void store4(E *p, const float *x) {  // 4 consecutive
    uint2 w;
    w.x = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
    w.y = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
    *reinterpret_cast<uint2 *>(p) = w;
  }
  static __device__ __forceinline__ void store8(E *p, const float *x) {
    store4(p, x);
    store4(p + 4, x + 4);
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
  static __device__ __forceinline__ floatx4 k32(floatx4 acc, const E *pa, int g, const BReg &b) {
    const float4 a0 = *reinterpret_cast<const float4 *>(pa + 8 * g);
    const float4 a1 = *reinterpret_cast<const float4 *>(pa + 8 * g + 4);
    const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = mfma_f32_k4(a[e], b.v[e], acc);
    return acc;
  }
  static __device__ __forceinline__ BReg breg_lds(const E *pb, int g) {
    const float4 b0 = *reinterpret_cast<const float4 *>(pb + 8 * g);
    const float4 b1 = *reinterpret_cast<const float4 *>(pb + 8 * g + 4);
    BReg b = {{b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w}};
    return b;
  }
  static __device__ __forceinline__ BReg breg_lds_scaled(const E *pb, int g, const float *sc) {
    BReg b = breg_lds(pb, g);
    const float4 s0 = *reinterpret_cast<const float4 *>(sc + 8 * g);
    const float4 s1 = *reinterpret_cast<const float4 *>(sc + 8 * g + 4);
    b.v[0] *= s0.x; b.v[1] *= s0.y; b.v[2] *= s0.z; b.v[3] *= s0.w;
    b.v[4] *= s1.x; b.v[5] *= s1.y; b.v[6] *= s1.z; b.v[7] *= s1.w;
    return b;
  }
  static __device__ __forceinline__ floatx4 k16_f32a(floatx4 acc, const float *pa, int g,
                                                     floatx4 t) {
    const float4 a4 = *reinterpret_cast<const float4 *>(pa + 4 * g);
    acc = mfma_f32_k4(a4.x, t[0], acc);
    acc = mfma_f32_k4(a4.y, t[1], acc);
    acc = mfma_f32_k4(a4.z, t[2], acc);
    acc = mfma_f32_k4(a4.w, t[3], acc);
    return acc;
  }
  static __device__ __forceinline__ floatx4 k16_ea(floatx4 acc, const E *pa, int g, floatx4 t) {
    return k16_f32a(acc, pa, g, t);
  }
  static __device__ __forceinline__ void store4(E *p, const float *x) {
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
  static __device__ __forceinline__ void store8(E *p, const float *x) {
    store4(p, x);
    store4(p + 4, x + 4);
  }
};

// FwdParams is declared in kda_launch.h

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
  return lo;
}

// Block column J of INV = (I + L)^-1 from the diagonal-block inverses T_II:
//   X_JJ = T_JJ,  X_IJ = -T_II sum_{K=J}^{I-1} L_IK X_KJ  (I > J),
// all tiles in registers (accumulator layout doubles as the 16x16x16 B operand).
// Stores INV Diag(beta) into INVb with the token axis permuted.
template <class Ar, int J, class Smem>
__device__ __forceinline__ void inv_block_column(Smem &sm, int g, int j) {
  floatx4 X[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) X[J][r] = Ar::tof(sm.Tdg[J][4 * g + r][j]);
#pragma unroll
  for (int I = J + 1; I < 4; ++I) {
    floatx4 R = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int K = J; K < I; ++K) R = Ar::k16_f32a(R, &sm.L[16 * I + j][16 * K], g, X[K]);
    floatx4 Y = {0.f, 0.f, 0.f, 0.f};
    Y = Ar::k16_ea(Y, &sm.Tdg[I][j][0], g, R);
    X[I] = -Y;
  }
  const float bj = sm.beta[16 * J + j];
#pragma unroll
  for (int I = J; I < 4; ++I) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      sm.INVb[16 * I + 4 * g + r][kperm(16 * J + j)] = Ar::cvt(X[I][r] * bj);
  }
}

// Recurrence operands of one token (8 channels) into LDS: K_decay and Q_decay
// rows, channels 8cg..8cg+7 = two groups of 4 consecutive permuted positions.
template <class Ar, class Smem>
__device__ __forceinline__ void write_phase2_row(Smem &sm, const float (&Kdec)[8],
                                                 const float (&Qdec)[8], int i, int cg) {
  Ar::store4(&sm.A.p2.Kd[i][kperm(8 * cg)], &Kdec[0]);
  Ar::store4(&sm.A.p2.Kd[i][kperm(8 * cg + 4)], &Kdec[4]);
  Ar::store4(&sm.A.p2.Qd[i][kperm(8 * cg)], &Qdec[0]);
  Ar::store4(&sm.A.p2.Qd[i][kperm(8 * cg + 4)], &Qdec[4]);
}
// K_restore^T for this thread's 4 tokens (consecutive permuted positions) x 8 channels.
template <class Ar, class Smem>
__device__ __forceinline__ void write_phase2_krt(Smem &sm, const float (&Kres)[4][8], int w,
                                                 int tq, int cg) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float x[4] = {Kres[0][c], Kres[1][c], Kres[2][c], Kres[3][c]};
    Ar::store4(&sm.A.p2.KrT[8 * cg + c][kperm(16 * w + 4 * tq)], x);
  }
}

template <typename Tin, bool F32C, int NT>
__global__ void __launch_bounds__(FWD_THREADS, 1) kda_fwd_kernel(FwdParams p) {
  using Ar = Arith<F32C>;
  using E = typename Ar::E;
  using BReg = typename Ar::BReg;
  constexpr bool ALIAS = F32C;  // fp32 operands: overlay phase 1 and phase 2 in LDS
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
      const int64_t ds = cu_at(p, doc);
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

  const Tin *__restrict__ q = (const Tin *)p.q;
  const Tin *__restrict__ k = (const Tin *)p.k;
  const Tin *__restrict__ v = (const Tin *)p.v;
  const Tin *__restrict__ z = (const Tin *)p.z;
  const Tin *__restrict__ bt = (const Tin *)p.beta;
  Tin *__restrict__ o = (Tin *)p.o;
  const float escale = __expf(p.A_log ? p.A_log[h] : 0.0f);
  const float g_min = p.g_min;

  // M_qk and INV Diag(beta) keep zero upper 16x16 blocks for the whole chain.
  for (int x = tid; x < CH * CH; x += FWD_THREADS) {
    (&sm.Mqk[0][0])[x] = Ar::cvt(0.f);
    (&sm.INVb[0][0])[x] = Ar::cvt(0.f);
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

  int64_t doc_end = (p.mode == 2) ? b : cu_at(p, doc + 1);

  // Raw inputs of one chunk.  Token indices are clamped into the chunk so every
  // load is unconditional (all in flight at once); rows past `len` are masked
  // after conversion.  The next chunk's loads are issued before the current
  // chunk's prep and recurrence, hiding HBM latency behind them.
  using IO = io<Tin>;
  typename IO::raw8 Rq[4], Rk[4], Rz[4];
  typename IO::raw1 Rv[4][NT][4], Rb;
  auto fetch = [&](int64_t c0, int n) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t tok = c0 + min(16 * w + 4 * tq + r, n - 1);
      const int64_t off = (tok * H + h) * (int64_t)D + 8 * cg;
      Rq[r] = IO::ld8(q + off);
      Rk[r] = IO::ld8(k + off);
      Rz[r] = IO::ld8(z + off);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n2 = 0; n2 < NT; ++n2)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t tok = c0 + min(16 * m + 4 * g + r, n - 1);
          const int vcol = m_cols ? j : colW + 16 * n2 + j;  // M columns read nothing useful
          Rv[m][n2][r] = IO::ld1(v + (tok * H + h) * (int64_t)D + vcol);
        }
    Rb = IO::ld1(bt + (c0 + min(tid & 63, n - 1)) * H + h);
  };
  int64_t pos = a;
  int len_next = (int)min((int64_t)CH, min(b, doc_end) - a);
  if (len_next > 0) fetch(a, len_next);
  while (pos < b) {
    const int64_t cs = pos;
    const int len = len_next;
    if (len <= 0) break;  // only if device and host offsets disagree; never loop forever

    // ================= prep (a1-a4) =================
    // a1: gate of z for tokens 16w + 4tq + r, channels 8cg..8cg+7 (q, k stay
    //     packed until a2 consumes them).
    float G[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool valid = 16 * w + 4 * tq + r < len;
      float zz[8];
      IO::cvt8(Rz[r], zz);
#pragma unroll
      for (int c = 0; c < 8; ++c) G[r][c] = valid ? kda_gate(zz[c], escale, g_min) : 0.f;
    }
    if (tid < CH) sm.beta[tid] = (tid < len) ? IO::cvt1(Rb) : 0.f;
    // V in accumulator layout (tokens 16m + 4g + r, this wave's columns)
    floatx4 Vt[4][NT];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          Vt[m][n][r] = (16 * m + 4 * g + r < len && !m_cols) ? IO::cvt1(Rv[m][n][r]) : 0.f;
    // where the next chunk starts (chunks restart at document starts); its
    // loads are issued once a2 has consumed the packed q and k
    int64_t npos, nlen;
    {
      npos = cs + len;
      int64_t nend = doc_end;
      if (p.mode != 2 && npos == doc_end && npos < b) nend = cu_at(p, doc_of(p.cu, p.N, npos) + 1);
      nlen = (npos < b) ? min((int64_t)CH, min(b, nend) - npos) : 0;
    }

    // inclusive cumulative sum over the chunk: in-lane over r, across the
    // 4 token groups of the wave (lanes 16 apart), then across waves.
    {
      float tot[8], x1[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        G[1][c] += G[0][c];
        G[2][c] += G[1][c];
        G[3][c] += G[2][c];
        tot[c] = G[3][c];
        const float up16 = __shfl_up(tot[c], 16);
        x1[c] = tot[c] + (tq >= 1 ? up16 : 0.f);
        const float up32 = __shfl_up(x1[c], 32);
        const float incl = x1[c] + (tq >= 2 ? up32 : 0.f);
        const float excl = incl - tot[c];
#pragma unroll
        for (int r = 0; r < 4; ++r) G[r][c] += excl;
      }
      if (tq == 3) {
#pragma unroll
        for (int c = 0; c < 8; ++c) sm.wtot[w][8 * cg + c] = G[3][c];
      }
    }
    __syncthreads();  // B1
    SCHED_FENCE();
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float t0 = sm.wtot[0][8 * cg + c], t1 = sm.wtot[1][8 * cg + c];
      const float t2 = sm.wtot[2][8 * cg + c];
      const float off = (w > 0 ? t0 : 0.f) + (w > 1 ? t1 : 0.f) + (w > 2 ? t2 : 0.f);
#pragma unroll
      for (int r = 0; r < 4; ++r) G[r][c] += off;
    }
    if (tq == 0) {
#pragma unroll
      for (int c = 0; c < 8; ++c) sm.Gref[w][8 * cg + c] = G[0][c];
    }
    if (w == 3 && tq == 3) {
#pragma unroll
      for (int c = 0; c < 8; ++c) sm.gamC[8 * cg + c] = G[3][c];  // log form for now
    }
    __syncthreads();  // B2
    SCHED_FENCE();

    // a2: subtile operands (phase 1) and recurrence operands (phase 2)
    float Kdec[4][8], Qdec[4][8], Kres[4][8];
    {
      float Pj[8], Rj[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float gref = sm.Gref[w][8 * cg + c];
        Pj[c] = __expf(gref);                              // e^(G_s)
        Rj[c] = __expf(sm.gamC[8 * cg + c] - gref);        // e^(G_C - G_s) <= 1
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * w + 4 * tq + r;
        const bool valid = i < len;
        float qv[8], kv[8], qh[8], kh[8], ki[8];
        IO::cvt8(Rq[r], qv);
        IO::cvt8(Rk[r], kv);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float e1 = __expf(G[r][c] - sm.Gref[w][8 * cg + c]);  // <= 1
          const float e2 = __builtin_amdgcn_rcpf(e1);                   // < e^75
          const float qq = valid ? qv[c] : 0.f, kk = valid ? kv[c] : 0.f;
          qh[c] = qq * e1;
          kh[c] = kk * e1;
          ki[c] = kk * e2;
          Qdec[r][c] = qh[c] * Pj[c];
          Kdec[r][c] = kh[c] * Pj[c];
          Kres[r][c] = ki[c] * Rj[c];
        }
        Ar::store8(&sm.A.p1.Qh[i][8 * cg], qh);
        Ar::store8(&sm.A.p1.Kh[i][8 * cg], kh);
        Ar::store8(&sm.A.p1.Ki[i][8 * cg], ki);
        if constexpr (!ALIAS) write_phase2_row<Ar>(sm, Kdec[r], Qdec[r], i, cg);
        SCHED_FENCE();
      }
      if constexpr (!ALIAS) write_phase2_krt<Ar>(sm, Kres, w, tq, cg);
      // F[pair][c] = e^(Gref[I][c] - Gref[J][c]), pairs (1,0),(2,0),(2,1),(3,0),(3,1),(3,2)
      for (int x = tid; x < 6 * D; x += FWD_THREADS) {
        const int pi = x / D, c = x % D;
        const int I = (pi == 0) ? 1 : (pi < 3 ? 2 : 3);
        const int J = (pi == 0) ? 0 : (pi < 3 ? pi - 1 : pi - 3);
        sm.F[pi][c] = __expf(sm.Gref[I][c] - sm.Gref[J][c]);
      }
    }
    SCHED_FENCE();
    if (nlen > 0) fetch(npos, (int)nlen);  // next chunk's inputs stream in behind this one
    len_next = (int)nlen;
    __syncthreads();  // B3
    SCHED_FENCE();

    // a3: A_qk and A_kk per subtile pair (I >= J); wave w takes pairs w, w+4, w+8.
    for (int pidx = w; pidx < 10; pidx += 4) {
      const int I = (pidx == 0) ? 0 : (pidx < 3 ? 1 : (pidx < 6 ? 2 : 3));
      const int J = pidx - I * (I + 1) / 2;
      floatx4 aq = {0.f, 0.f, 0.f, 0.f}, ak = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        BReg bk;
        if (I == J) {
          bk = Ar::breg_lds(&sm.A.p1.Ki[16 * J + j][32 * kb], g);
        } else {
          const int fp = I * (I - 1) / 2 + J;
          bk = Ar::breg_lds_scaled(&sm.A.p1.Ki[16 * J + j][32 * kb], g, &sm.F[fp][32 * kb]);
        }
        aq = Ar::k32(aq, &sm.A.p1.Qh[16 * I + j][32 * kb], g, bk);
        ak = Ar::k32(ak, &sm.A.p1.Kh[16 * I + j][32 * kb], g, bk);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ii = 4 * g + r;  // row inside subtile I; column j inside subtile J
        const bool keep_q = (I > J) || (j <= ii);
        const bool keep_k = (I > J) || (j < ii);
        sm.Mqk[16 * I + ii][kperm(16 * J + j)] = Ar::cvt(keep_q ? aq[r] : 0.f);
        sm.L[16 * I + ii][16 * J + j] = keep_k ? sm.beta[16 * I + ii] * ak[r] : 0.f;
      }
    }
    __syncthreads();  // B4: phase-1 operands dead, L complete
    SCHED_FENCE();

    // phase 2 operands into the LDS region phase 1 occupied
    if constexpr (ALIAS) {
#pragma unroll
      for (int r = 0; r < 4; ++r) write_phase2_row<Ar>(sm, Kdec[r], Qdec[r], 16 * w + 4 * tq + r, cg);
      write_phase2_krt<Ar>(sm, Kres, w, tq, cg);
    }
    // a4 (i): inverse of the diagonal block J = w of I + L, one column per lane
    if (lane < 16) {
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = (r == lane) ? 1.f : 0.f;
#pragma unroll
        for (int s = 0; s < r; ++s) acc = fmaf(-sm.L[16 * w + r][16 * w + s], x[s], acc);
        x[r] = acc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.Tdg[w][r][lane] = Ar::cvt(x[r]);
    }
    __syncthreads();  // B5
    SCHED_FENCE();

    if (w == 3 && tq == 3) {  // gamma^C from its log (read by the recurrence after B6)
#pragma unroll
      for (int c = 0; c < 8; ++c) sm.gamC[8 * cg + c] = __expf(G[3][c]);
    }
    // a4 (ii): block column J = w of INV: X_IJ = -T_II sum_{K=J}^{I-1} L_IK X_KJ
    switch (w) {
      case 0: inv_block_column<Ar, 0>(sm, g, j); break;
      case 1: inv_block_column<Ar, 1>(sm, g, j); break;
      case 2: inv_block_column<Ar, 2>(sm, g, j); break;
      default: inv_block_column<Ar, 3>(sm, g, j); break;
    }
    __syncthreads();  // B6
    SCHED_FENCE();

    // ================= recurrence (a5) =================
    BReg sb[4][NT];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int n = 0; n < NT; ++n) sb[kb][n] = Ar::breg(S[2 * kb][n], S[2 * kb + 1][n]);

    floatx4 U[4][NT];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        floatx4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) x = Ar::k32(x, &sm.A.p2.Kd[16 * m + j][32 * kb], g, sb[kb][n]);
        U[m][n] = Vt[m][n] - x;  // B' = V - K_decay S (Diag(beta) is folded into INV)
      }
    SCHED_FENCE();
    BReg bb[2][NT];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int n = 0; n < NT; ++n) bb[kb][n] = Ar::breg(U[2 * kb][n], U[2 * kb + 1][n]);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        floatx4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb <= (m >> 1); ++kb)
          x = Ar::k32(x, &sm.INVb[16 * m + j][32 * kb], g, bb[kb][n]);
        U[m][n] = x;
      }
    SCHED_FENCE();
    BReg ub[2][NT];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int n = 0; n < NT; ++n) ub[kb][n] = Ar::breg(U[2 * kb][n], U[2 * kb + 1][n]);

    // O = Q_decay S + M_qk U  (off the serial state path)
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        floatx4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) x = Ar::k32(x, &sm.A.p2.Qd[16 * m + j][32 * kb], g, sb[kb][n]);
#pragma unroll
        for (int kb = 0; kb <= (m >> 1); ++kb)
          x = Ar::k32(x, &sm.Mqk[16 * m + j][32 * kb], g, ub[kb][n]);
        if (p.mode != 2) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 16 * m + 4 * g + r;
            if (i < len) io<Tin>::store1(o + ((cs + i) * H + h) * (int64_t)D + colW + 16 * n + j, x[r]);
          }
        }
      }
    SCHED_FENCE();
    // S <- Diag(gamma^C) S + K_restore^T U
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float4 gc = *reinterpret_cast<const float4 *>(&sm.gamC[16 * m + 4 * g]);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        floatx4 x = S[m][n];
        x[0] *= gc.x; x[1] *= gc.y; x[2] *= gc.z; x[3] *= gc.w;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) x = Ar::k32(x, &sm.A.p2.KrT[16 * m + j][32 * kb], g, ub[kb][n]);
        S[m][n] = x;
      }
    }

    SCHED_FENCE();
    pos += len;
    if (p.mode == 2) {
      if (pos == b)  // emit the pair [S~ | M] for this segment
        state_store(S, p.final_state + ((int64_t)item * H + h) * (D * 2 * D), 2 * D, colW, g, j);
    } else if (pos == doc_end) {
      // document boundary: emit its final state, then reset for the next document
      if (p.final_state) state_store(S, p.final_state + ((int64_t)doc * H + h) * (D * D), D, colW, g, j);
      if (pos < b) {
        doc = doc_of(p.cu, p.N, pos);
        doc_end = cu_at(p, doc + 1);
        if (p.doc_init) {
          state_load(S, p.doc_init + ((int64_t)doc * H + h) * (D * D), D, colW, g, j);
        } else {
#pragma unroll
          for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int n = 0; n < NT; ++n) S[m][n] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    __syncthreads();  // B7: LDS reuse by the next chunk
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

template <typename Tin, bool F32C, int NT>
static hipError_t launch_fwd_t(const FwdParams &p, hipStream_t stream) {
  const int units = p.n_items * p.H;
  const int groups = (units + 7) / 8;
  const dim3 grid((unsigned)(groups * 8 * p.nsplit));
  hipLaunchKernelGGL((kda_fwd_kernel<Tin, F32C, NT>), grid, dim3(FWD_THREADS), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_fwd(FwdParams p, bool bf16_in, bool f32_compute, hipStream_t stream) {
  // slices of 64 state columns per (item, head), 16 per wave: two for the
  // 128 value columns, four for the [S~ | M] pair columns
  p.nsplit = (p.mode == 2) ? 4 : 2;
  if (bf16_in)
    return f32_compute ? launch_fwd_t<bf16_t, true, 1>(p, stream)
                       : launch_fwd_t<bf16_t, false, 1>(p, stream);
  return f32_compute ? launch_fwd_t<float, true, 1>(p, stream)
                     : launch_fwd_t<float, false, 1>(p, stream);
}

hipError_t launch_copy_empty(const int32_t *cu, int64_t T, const float *init, float *fin, int N,
                             int H, hipStream_t stream) {
  hipLaunchKernelGGL(kda_copy_empty_kernel, dim3((unsigned)(N * H)), dim3(256), 0, stream, cu, T,
                     init, fin, H);
  return hipGetLastError();
}

}  // namespace kda
