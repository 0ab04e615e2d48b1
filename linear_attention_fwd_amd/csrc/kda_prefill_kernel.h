// kda_prefill_kernel.h -- the fused chunkwise KDA prefill kernel (no workspace),
// included by kda_prefill.hip (bounded gate, inputs as given) and by
// kda_prefill_ext.hip (the unbounded gate and raw inputs), so that each
// translation unit instantiates its own variants.
//
// One workgroup (4 waves) runs the serial chunk chain of one (item, head,
// 64-column slice of the state).  An item is a document of the packed sequence
// (mode 0), or a fixed token range that may contain document starts: a segment
// re-run from its scanned entry state (mode 1) or a segment pair (M, S~) built
// from a zero state (mode 2).  Per chunk of C = 64 tokens the workgroup runs
// the prep stages a1-a4 of kda_chunk.h (token-parallel, all waves; the "chunk
// prep" of the pages) into LDS, then the recurrence a5 (each wave owns 16
// state columns, S held in fp32 MFMA accumulators for the whole chain).
//
// Arithmetic: bf16 MFMA operands with fp32 accumulation (F32C = false) or an
// fp32-MFMA verification build (F32C = true) from the same source.
#pragma once
#include "kda_chunk.h"

namespace kda {

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
  E L[CH * CH];      // strict lower part used
  E Tdg[4][SUB * SUB];  // inverses of the diagonal 16x16 blocks of I + L
  float gamC[D];        // gamma^C = e^(G_C)
  PrepLds ps;
};

// Recurrence operands of one token (8 channels) into LDS: K_decay and Q_decay
// rows, channels 8cg..8cg+7 = two groups of 4 consecutive permuted positions.
template <class Ar, class Smem>
__device__ __forceinline__ void write_phase2_row(Smem &sm, const float *Kdec, const float *Qdec,
                                                 int i, int cg) {
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

// UNB: the unbounded Kimi Linear gate (diagonal subtiles whose decay range is
// too wide for two factors are formed per position, prep_diag_positions);
// RAW: q, k unnormalised and beta a logit (normalised and sigmoid applied here).
template <typename Tin, bool F32C, bool UNB, bool RAW>
__global__ void __launch_bounds__(FWD_THREADS, 1) kda_fwd_kernel(FwdParams p) {
  using Ar = Arith<F32C>;
  using E = typename Ar::E;
  using IO = bufio<Tin>;
  using TC = Tile<E, CH>;   // 128 x 64 and 64 x 64 operand tiles
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
  const int colW = split * 64 + w * 16;  // first state column of this wave
  const int H = p.H;

  int64_t a, b;
  int doc;
  // mode 2: slices 0,1 carry S~ (value columns), slices 2,3 carry M (identity start, v = 0)
  const bool m_cols = (p.mode == 2) && (colW >= D);
  const float *init_src = nullptr;  // initial state (row-major D x D), nullptr = 0 / identity
  if (p.mode == 0) {
    a = cu_at(p.cu, p.T, item);
    b = cu_at(p.cu, p.T, item + 1);
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
      const int64_t ds = uni64(cu_at(p.cu, p.T, doc));
      if (ds > a) {
        if (m_cols) {
          float *dst = p.final_state + ((int64_t)item * H + h) * (D * 2 * D);
          for (int x = tid; x < D * 64; x += FWD_THREADS)
            dst[(x / 64) * (2 * D) + split * 64 + x % 64] = 0.f;
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

  // ---- initial state, in accumulator layout: S[m] holds rows 16m+4g+r,
  //      column colW + j --------------------------------------------------
  floatx4 S[8];
  if (m_cols) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) S[m][r] = (16 * m + 4 * g + r == colW + j - D) ? 1.f : 0.f;
  } else if (init_src) {
    state_load(S, init_src, D, colW, g, j);
  } else {
#pragma unroll
    for (int m = 0; m < 8; ++m) S[m] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  int64_t doc_end = (p.mode == 2) ? b : uni64(cu_at(p.cu, p.T, doc + 1));

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
      if (p.mode != 2 && npos == doc_end && npos < b)
        nend = uni64(cu_at(p.cu, p.T, doc_of(p.cu, p.N, npos) + 1));
      nlen = (npos < b) ? min((int64_t)CH, min(b, nend) - npos) : 0;
    }

    if constexpr (RAW) {  // q and k rows to unit L2 norm
      l2norm_rows(Rq);
      l2norm_rows(Rk);
    }
    float G[4][8];
    prep_gate_cumsum<IO, UNB>(sm.ps, Rz, Rb, c1, gmin2, len, tid, w, tq, cg, G, RAW);  // two barriers
    if constexpr (UNB) {
      static_assert(sizeof(sm.A.p1) >= 4 * diag_stage_bytes<IO>(),
                    "per-wave staging for the diagonal subtiles");
      if (!diag_two_factor(sm.ps, w))  // else the subtile products form it
        prep_diag_positions<IO, Ar>(reinterpret_cast<char *>(&sm.A.p1) + w * diag_stage_bytes<IO>(),
                                    Rq, Rk, G, sm.ps.beta, sm.L, w, tq, cg,
                                    [&](int row, int col, float m) {
                                      sm.Mqk[TC::idx(row, kperm(col))] = Ar::cvt(m);
                                    });
      __syncthreads();  // the staging area becomes the subtile operand tiles
      SCHED_FENCE();
    }

    float Kres[4][8];
    float Kdec_s[4][8], Qdec_s[4][8];  // fp32 build: held until phase 1 is consumed
    prep_decay_operands<Ar, IO, UNB>(sm.ps, sm.A.p1.Qh,
                                [&](int, int i, const float *kh) {
                                  using TD = Tile<typename Ar::E, D>;
                                  Ar::store4(&sm.A.p1.Kh[TD::idx(i, 8 * cg)], kh);
                                  Ar::store4(&sm.A.p1.Kh[TD::idx(i, 8 * cg + 4)], kh + 4);
                                },
                                sm.A.p1.Ki, Rq, Rk, G, w, tq, cg, Kres,
                                [&](int i, const float *kdec, const float *qdec) {
                                  if constexpr (!ALIAS) {
                                    write_phase2_row<Ar>(sm, kdec, qdec, i, cg);
                                  } else {
                                    const int r = i & 3;
#pragma unroll
                                    for (int c = 0; c < 8; ++c) {
                                      Kdec_s[r][c] = kdec[c];
                                      Qdec_s[r][c] = qdec[c];
                                    }
                                  }
                                });
    if constexpr (!ALIAS) write_phase2_krt<Ar>(sm, Kres, w, tq, cg);
    prep_pair_factors<UNB>(sm.ps, tid);
    if (tid < D) sm.gamC[tid] = __builtin_amdgcn_exp2f(sm.ps.GC2[tid]);
    SCHED_FENCE();
    if (nlen > 0) fetch(npos, (int)nlen);  // next chunk's inputs stream in behind this one
    len_next = (int)nlen;
    __syncthreads();  // B3
    SCHED_FENCE();

    prep_subtile_products<Ar, PROD_MQK | PROD_L, UNB>(sm.ps, sm.A.p1.Qh, sm.A.p1.Kh, sm.A.p1.Ki, sm.L, w, g, j,
                              [&](int row, int J, const float *mq) {
                                Ar::store4(&sm.Mqk[TC::idx(row, kperm(16 * J + 4 * g))], mq);
                              });
    __syncthreads();  // B4: phase-1 operands dead, L complete
    SCHED_FENCE();

    if constexpr (ALIAS) {  // phase 2 operands into the LDS region phase 1 occupied
#pragma unroll
      for (int r = 0; r < 4; ++r) write_phase2_row<Ar>(sm, Kdec_s[r], Qdec_s[r], 16 * w + 4 * tq + r, cg);
      write_phase2_krt<Ar>(sm, Kres, w, tq, cg);
    }
    const floatx4 Tww = prep_diag_inverse<Ar>(sm.L, sm.Tdg, w, g, j);
    __syncthreads();  // B5
    SCHED_FENCE();
    prep_block_columns<Ar>(sm.L, sm.Tdg, sm.ps.beta, sm.INVb, Tww, w, g, j);
    __syncthreads();  // B6
    SCHED_FENCE();

    // ================= recurrence (a5) =================
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(o + (cs * H + h) * D, p.mode != 2 ? ((len - 1) * H + 1) * D * ES : 0);
    chunk_recurrence<Ar, IO>(sm.A.p2.Kd, sm.A.p2.Qd, sm.A.p2.KrT, sm.Mqk, sm.INVb, sm.gamC, S, Vt,
                             p.mode != 2, ro, off_v, rowb, g, j);

    pos += len;
    if (p.mode == 2) {
      if (pos == b)  // emit the pair [S~ | M] for this segment
        state_store(S, uniptr(p.final_state + ((int64_t)item * H + h) * (D * 2 * D)), 2 * D, colW, g, j);
    } else if (pos == doc_end) {
      // document boundary: emit its final state, then reset for the next document
      if (p.final_state)
        state_store(S, uniptr(p.final_state + ((int64_t)doc * H + h) * (D * D)), D, colW, g, j);
      if (pos < b) {
        doc = doc_of(p.cu, p.N, pos);
        doc_end = uni64(cu_at(p.cu, p.T, doc + 1));
        if (p.doc_init) {
          state_load(S, uniptr(p.doc_init + ((int64_t)doc * H + h) * (D * D)), D, colW, g, j);
        } else {
#pragma unroll
          for (int m = 0; m < 8; ++m) S[m] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    // The next chunk writes beta, wtot, Gref, GC2 before touching anything the
    // recurrence reads, except with overlaid operands (ALIAS), where phase 1
    // of the next chunk overwrites phase 2 of this one.
    if constexpr (ALIAS) __syncthreads();  // B7
  }
}

template <typename Tin, bool F32C, bool UNB, bool RAW>
inline hipError_t launch_fwd_t(const FwdParams &p, hipStream_t stream) {
  const int units = p.n_items * p.H;
  const int groups = (units + 7) / 8;
  const dim3 grid((unsigned)(groups * 8 * p.nsplit));
  hipLaunchKernelGGL((kda_fwd_kernel<Tin, F32C, UNB, RAW>), grid, dim3(FWD_THREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kda
