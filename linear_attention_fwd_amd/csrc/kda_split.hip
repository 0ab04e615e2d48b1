// kda_split.hip -- two-kernel chunkwise KDA prefill for gfx950 (bf16 operands).
//
// The chunk prep (stages a1-a4 of kda_chunk.h) depends only on the chunk's own
// tokens, so it runs token-parallel over every (head, chunk) at once: one
// workgroup per chunk, two workgroups per compute unit.  It writes the
// recurrence operands of its chunk, the "chunk image", to a workspace in the
// exact layout of the recurrence kernel's LDS tiles.  The recurrence kernel
// then runs the serial chain of each (document, head, 64-column slice) and
// only streams images: global -> LDS copies into a double buffer, one chunk
// ahead of the MFMA work and issued by waves of their own, with the lines of a
// later chunk pulled into L2 before that (the split into a
// prep kernel and a recurrence kernel is the FlashKDA structure of the
// SemiAnalysis page, section "FlashKDA 算法").
//
// Chunks restart at every document start; chunk k of document d has slot
// first_slot(d) + k (kda_launch.h), the images of head h lie at
// ws + (h * n_slots + slot) * sizeof(ChunkImage).
#include <stddef.h>

#include "kda_chunk.h"

namespace kda {

// M_qk and INV Diag(beta) as the recurrence reads them: its 32-wide k steps
// over rows 0..31 stop at column 31, so the top-right 32 x 32 quarter is never
// read and is not stored.  Rows 0..31 are 32 wide, rows 32..63 are 64 wide,
// each part XOR-swizzled like Tile (token axis permuted, see kperm).
struct PackedLower {
  using Top = Tile<bf16_t, 32>;
  using Bot = Tile<bf16_t, 64>;
  static constexpr int TOP = 32 * 32;
  static constexpr int ELEMS = TOP + 32 * 64;
  // element offset of logical (r, col); col < 32 when r < 32
  static __device__ __forceinline__ int idx(int r, int col) {
    return r < 32 ? Top::idx(r, col) : TOP + Bot::idx(r - 32, col);
  }
};

// Recurrence operands of one (head, chunk), laid out as LDS tiles.
struct __align__(16) ChunkImage {
  bf16_t Kd[CH * D];                 // K_decay, channel axis permuted
  bf16_t Qd[CH * D];                 // Q_decay, channel axis permuted
  bf16_t KrT[D * CH];                // K_restore^T, token axis permuted
  bf16_t Mqk[PackedLower::ELEMS];    // M_qk
  bf16_t INVb[PackedLower::ELEMS];   // INV Diag(beta)
  float gamC[D];                     // gamma^C
  float pad[128];                    // the image is a whole number of 1 KB copy blocks
};
constexpr int IMG_BYTES = (int)sizeof(ChunkImage);
constexpr int IMG_BLOCKS = IMG_BYTES / 1024;
static_assert(IMG_BYTES % 1024 == 0, "chunk image must be whole 1 KB blocks");
static_assert(IMG_BYTES == CHUNK_IMAGE_BYTES, "workspace formula of kda_launch.h");
static_assert(offsetof(ChunkImage, Qd) % 1024 == 0 && offsetof(ChunkImage, KrT) % 1024 == 0 &&
                  offsetof(ChunkImage, Mqk) % 1024 == 0 && offsetof(ChunkImage, INVb) % 1024 == 0,
              "operand tiles must start on copy-block boundaries");
constexpr int OFF_KD = (int)offsetof(ChunkImage, Kd);
constexpr int OFF_QD = (int)offsetof(ChunkImage, Qd);
constexpr int OFF_KRT = (int)offsetof(ChunkImage, KrT);
constexpr int OFF_MQK = (int)offsetof(ChunkImage, Mqk);
constexpr int OFF_INVB = (int)offsetof(ChunkImage, INVb);
constexpr int OFF_GAMC = (int)offsetof(ChunkImage, gamC);

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
// 4 consecutive bf16 (8 bytes) into the image at byte offset off
__device__ __forceinline__ void img_st4(__amdgpu_buffer_rsrc_t r, int off, const float *x) {
  const bf16x4 v = to_bf16x4(floatx4{x[0], x[1], x[2], x[3]});
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// Prep: one workgroup per (chunk slot, head).
// ---------------------------------------------------------------------------
// 51 KB, so that three workgroups share a compute unit: the query- and
// key-side subtile operands take turns in one tile (M_qk is formed first, then
// the key side, held in registers meanwhile, overwrites the query side for L).
struct __align__(16) PrepSmem {
  union {
    struct {
      bf16_t QKh[CH * D];  // q_i e^(G_i - G_s(i)), then k_i e^(G_i - G_s(i))
      bf16_t Ki[CH * D];   // k_j e^(G_s(j) - G_j)
    } p1;
    bf16_t INVb[CH * CH];  // staged after the subtile operands are dead
  } u;
  bf16_t L[CH * CH];
  bf16_t Tdg[4][SUB * SUB];
  PrepLds ps;
};
static_assert(3 * sizeof(PrepSmem) <= 160 * 1024, "three prep workgroups per compute unit");

// UNB: the unbounded Kimi Linear gate; the diagonal subtiles of M_qk and L are
// then formed per position (prep_diag_positions) and the off-diagonal ones
// with the key side referenced to the end of its subtile.  RAW: q, k
// unnormalised and beta a logit (normalised and sigmoid applied here).
template <bool UNB, bool RAW>
__global__ void __launch_bounds__(FWD_THREADS, 3) kda_chunk_prep_kernel(SplitParams p) {
  using Ar = Arith<false>;
  using IO = bufio<bf16_t>;
  using TD = Tile<bf16_t, D>;
  using TC = Tile<bf16_t, CH>;
  constexpr int ES = 2;
  __shared__ PrepSmem sm;

  const int H = p.H;
  const int h = blockIdx.x % H;
  const int64_t slot = blockIdx.x / H;
  const int d = doc_of_slot(p.cu, p.N, slot);
  const int64_t a = uni64(cu_at(p.cu, p.T, d));
  const int64_t b = uni64(cu_at(p.cu, p.T, d + 1));
  const int64_t cs = a + (slot - first_slot(a, d)) * CH;
  if (cs >= b) return;  // no chunk maps to this slot
  const int len = (int)min((int64_t)CH, b - cs);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int g = lane >> 4;
  const int j = lane & 15;
  const int tq = lane >> 4;
  const int cg = lane & 15;

  const bf16_t *q = (const bf16_t *)p.q;
  const bf16_t *k = (const bf16_t *)p.k;
  const bf16_t *z = (const bf16_t *)p.z;
  const bf16_t *bt = (const bf16_t *)p.beta;
  const float c1 = -__expf(p.A_log ? p.A_log[h] : 0.0f) * LOG2E;
  const float gmin2 = p.g_min * LOG2E;
  const int rowb = H * D * ES;

  // inputs of this chunk: tokens 16w + 4tq + r, channels 8cg..8cg+7; rows past
  // len read as 0 (bounded descriptors)
  typename IO::raw8 Rq[4], Rk[4], Rz[4];
  typename IO::raw1 Rb;
  {
    const int bytes = ((len - 1) * H + 1) * D * ES;
    const int64_t e0 = (cs * H + h) * D;
    const int off = ((16 * w + 4 * tq) * H * D + 8 * cg) * ES;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + e0, bytes);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + e0, bytes);
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(z + e0, bytes);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      Rz[r] = IO::ld8(rz, off + r * rowb);
      Rq[r] = IO::ld8(rq, off + r * rowb);
      Rk[r] = IO::ld8(rk, off + r * rowb);
    }
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(bt + (cs * H + h), ((len - 1) * H + 1) * ES);
    Rb = IO::ld1(rb, lane * H * ES);
  }

  if constexpr (RAW) {  // q and k rows to unit L2 norm
    l2norm_rows(Rq);
    l2norm_rows(Rk);
  }
  float G[4][8];
  prep_gate_cumsum<IO, UNB>(sm.ps, Rz, Rb, c1, gmin2, len, tid, w, tq, cg, G, RAW);  // two barriers

  const __amdgpu_buffer_rsrc_t ri =
      make_rsrc((char *)p.ws + ((int64_t)h * p.n_slots + slot) * IMG_BYTES, IMG_BYTES);
  if constexpr (UNB) {
    static_assert(sizeof(sm.u) >= 4 * diag_stage_bytes<IO>(), "per-wave staging for the diagonal subtiles");
    if (!diag_two_factor(sm.ps, w))  // else the subtile products form it
      prep_diag_positions<IO, Ar>(reinterpret_cast<char *>(&sm.u) + w * diag_stage_bytes<IO>(), Rq, Rk, G, sm.ps.beta, sm.L,
                        w, tq, cg, [&](int row, int col, float m) {
                          __builtin_amdgcn_raw_buffer_store_b16(
                              f32_to_bf16(m), ri, OFF_MQK + 2 * PackedLower::idx(row, kperm(col)), 0, 0);
                        });
    __syncthreads();  // the staging area becomes the subtile operand tiles
    SCHED_FENCE();
  }
  float Kres[4][8];
  bf16x4 kh_keep[4][2];  // key-side subtile operand of this thread's 4 tokens x 8 channels
  prep_decay_operands<Ar, IO, UNB>(sm.ps, sm.u.p1.QKh,
                              [&](int r, int, const float *kh) {
                                kh_keep[r][0] = to_bf16x4(floatx4{kh[0], kh[1], kh[2], kh[3]});
                                kh_keep[r][1] = to_bf16x4(floatx4{kh[4], kh[5], kh[6], kh[7]});
                              },
                              sm.u.p1.Ki, Rq, Rk, G, w, tq, cg, Kres,
                              [&](int i, const float *kdec, const float *qdec) {
                                const int c0 = 2 * TD::idx(i, kperm(8 * cg));
                                const int c1b = 2 * TD::idx(i, kperm(8 * cg + 4));
                                img_st4(ri, OFF_KD + c0, kdec);
                                img_st4(ri, OFF_KD + c1b, kdec + 4);
                                img_st4(ri, OFF_QD + c0, qdec);
                                img_st4(ri, OFF_QD + c1b, qdec + 4);
                              });
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float x[4] = {Kres[0][c], Kres[1][c], Kres[2][c], Kres[3][c]};
    img_st4(ri, OFF_KRT + 2 * TC::idx(8 * cg + c, kperm(16 * w + 4 * tq)), x);
  }
  prep_pair_factors<UNB>(sm.ps, tid);
  if (tid < D) buf_st_f32(ri, __builtin_amdgcn_exp2f(sm.ps.GC2[tid]), OFF_GAMC + 4 * tid);
  __syncthreads();
  SCHED_FENCE();

  prep_subtile_products<Ar, PROD_MQK, UNB>(sm.ps, sm.u.p1.QKh, nullptr, sm.u.p1.Ki, sm.L, w, g, j,
                                      [&](int row, int J, const float *mq) {
                                        img_st4(ri, OFF_MQK + 2 * PackedLower::idx(row, kperm(16 * J + 4 * g)), mq);
                                      });
  __syncthreads();  // the query side is consumed
  SCHED_FENCE();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 16 * w + 4 * tq + r;
    *reinterpret_cast<bf16x4 *>(&sm.u.p1.QKh[TD::idx(i, 8 * cg)]) = kh_keep[r][0];
    *reinterpret_cast<bf16x4 *>(&sm.u.p1.QKh[TD::idx(i, 8 * cg + 4)]) = kh_keep[r][1];
  }
  __syncthreads();
  SCHED_FENCE();
  prep_subtile_products<Ar, PROD_L, UNB>(sm.ps, nullptr, sm.u.p1.QKh, sm.u.p1.Ki, sm.L, w, g, j,
                                    [](int, int, const float *) {});
  // The recurrence reads the upper blocks (0,1) and (2,3) of M_qk and INV Diag(beta)
  // (its 32-wide k steps span two subtiles); they must hold zeros.
  const float zero4[4] = {0.f, 0.f, 0.f, 0.f};
  if (w & 1) img_st4(ri, OFF_MQK + 2 * PackedLower::idx(16 * (w - 1) + j, kperm(16 * w + 4 * g)), zero4);
  __syncthreads();  // subtile operands dead, L complete
  SCHED_FENCE();

  const floatx4 Tww = prep_diag_inverse<Ar>(sm.L, sm.Tdg, w, g, j);
  if (w & 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.u.INVb[TC::idx(16 * (w - 1) + 4 * g + r, kperm(16 * w + j))] = 0;
  }
  __syncthreads();
  SCHED_FENCE();
  prep_block_columns<Ar>(sm.L, sm.Tdg, sm.ps.beta, sm.u.INVb, Tww, w, g, j);
  __syncthreads();
  SCHED_FENCE();
  // INV Diag(beta): staged 64 x 64 tile -> packed image, one 16-byte chunk
  // (8 consecutive logical columns) per lane
  for (int x = tid; x < PackedLower::ELEMS / 8; x += FWD_THREADS) {
    int r, lc;  // logical row and chunk stored at packed chunk x
    if (x < PackedLower::TOP / 8) {
      r = x / 4;
      lc = (x % 4) ^ PackedLower::Top::sw(r);
    } else {
      r = 32 + (x - PackedLower::TOP / 8) / 8;
      lc = ((x - PackedLower::TOP / 8) % 8) ^ PackedLower::Bot::sw(r - 32);
    }
    const u32x4 v = *reinterpret_cast<const u32x4 *>(&sm.u.INVb[TC::idx(r, 8 * lc)]);
    __builtin_amdgcn_raw_buffer_store_b128(v, ri, OFF_INVB + 16 * x, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Recurrence: one workgroup per (item, head, column slice).  A workgroup has 8
// waves: waves 0..3 compute, waves 4..7 only copy the next chunk's image and v
// rows into the LDS double buffer and pull later chunks into L2.  A wave
// stalls while its copies queue up; with the roles split, those stalls fall on
// the copy wave of each SIMD while the compute wave keeps its MFMA work going.
//
// A compute wave owns NT tiles of 16 state columns, so a workgroup owns 64 NT
// columns.  Every workgroup copies the whole image of each chunk, whatever its
// column count, and that copy bounds the time per chunk; so where NT = 2
// workgroups (one per (item, head) unit, two for a segment pair's 256 columns)
// would leave compute units idle, NT = 1 spreads each unit over two
// workgroups (four for pairs), and where they fill the device, NT = 2 halves
// the number of chunk steps.  The
// workgroups of one unit share an XCD (blockIdx % 8), so the image reaches
// them from one L2.
// ---------------------------------------------------------------------------
constexpr int REC_COMPUTE_WAVES = 4;
constexpr int REC_COPY_WAVES = 4;
constexpr int REC_THREADS = 64 * (REC_COMPUTE_WAVES + REC_COPY_WAVES);
constexpr int REC_COPY_THREADS = 64 * REC_COPY_WAVES;
template <int NT> struct __align__(16) RecSmem {
  static constexpr int SLICE = 64 * NT;  // state columns per workgroup
  ChunkImage buf[2];
  bf16_t V[2][CH * SLICE];  // v rows of the chunk, this workgroup's columns
  uint32_t sink[64];        // destination of the L2 prefetch touches; never read
};
static_assert(sizeof(RecSmem<2>) <= 160 * 1024, "recurrence LDS exceeds a compute unit");

__device__ __forceinline__ bf16x8 frag(const bf16_t *tile, int idx) {
  return *reinterpret_cast<const bf16x8 *>(tile + idx);
}
__device__ __forceinline__ bf16x8 pack_tiles(floatx4 t0, floatx4 t1) {
  return to_bf16x8(floatx8{t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]});
}

// Registers one chunk step carries from phase to phase: S packed to bf16 (the
// B operand of the U' and O products), U, and U packed to bf16.
template <int NT> struct RecRegs {
  bf16x8 sb[NT][4];
  floatx4 U[NT][4];
  bf16x8 ub[NT][2];
};

// The chunk recurrence (chunk_recurrence in kda_chunk.h) for this wave's NT
// tiles of 16 state columns, operands from the chunk image in LDS, in four
// phases that each read one part of the image:
//   0: U' = V - K_decay S            (K_decay, V)
//   1: U = INV Diag(beta) U'         (INV Diag(beta))
//   2: O = Q_decay S + M_qk U        (Q_decay, M_qk)
//   3: S <- Diag(gamma^C) S + K_restore^T U   (K_restore^T, gamma^C)
// Each phase reads its MFMA A-operand fragments in one batch (lane (g, j): row
// 16m + j, k elements 32kb + 8g .. +7) and applies them to every tile.  The
// fragments read per batch are the whole phase for one tile, one 16-row block
// at a time for two (each fragment then feeds twice the MFMA work, and the
// whole-phase batches would not fit the register budget).
// V: the v rows of the chunk in LDS (vld elements per row), tile t of this
// wave at column vcol + 16 t.
template <int NT>
__device__ __forceinline__ void rec_phase0(const ChunkImage &im, const floatx4 (&S)[NT][8],
                                           const bf16_t *V, int vld, int vcol, int g, int j,
                                           RecRegs<NT> &R) {
  using TD = Tile<bf16_t, D>;
  constexpr int MB = NT == 1 ? 4 : 1;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) R.sb[t][kb] = pack_tiles(S[t][2 * kb], S[t][2 * kb + 1]);
#pragma unroll
  for (int m0 = 0; m0 < 4; m0 += MB) {
    bf16x8 kd[MB][4];
#pragma unroll
    for (int mm = 0; mm < MB; ++mm)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) kd[mm][kb] = frag(im.Kd, TD::idx(16 * (m0 + mm) + j, 32 * kb + 8 * g));
#pragma unroll
    for (int mm = 0; mm < MB; ++mm)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int m = m0 + mm;
        floatx4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) x = mfma_bf16_k32(kd[mm][kb], R.sb[t][kb], x);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          R.U[t][m][r] = bf16_to_f32(V[(16 * m + 4 * g + r) * vld + vcol + 16 * t + j]) - x[r];
      }
  }
}

template <int NT>
__device__ __forceinline__ void rec_phase1(const ChunkImage &im, int g, int j, RecRegs<NT> &R) {
  using PL = PackedLower;
  bf16x8 inv[6];
  int x = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int kb = 0; kb <= (m >> 1); ++kb, ++x) inv[x] = frag(im.INVb, PL::idx(16 * m + j, 32 * kb + 8 * g));
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    bf16x8 bb[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) bb[kb] = pack_tiles(R.U[t][2 * kb], R.U[t][2 * kb + 1]);
    x = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb <= (m >> 1); ++kb, ++x) acc = mfma_bf16_k32(inv[x], bb[kb], acc);
      R.U[t][m] = acc;
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) R.ub[t][kb] = pack_tiles(R.U[t][2 * kb], R.U[t][2 * kb + 1]);
}

// O = Q_decay S + M_qk U, formed transposed: with the operands of each product
// swapped, lane (g, j) ends up with token 16m + j, columns 4g..4g+3 of the
// tile and stores them with one 8-byte write through the bounded descriptor
// ro (tokens past the chunk are dropped) at byte offset off_o + token * rowb +
// 32 t, off_o = (j * H * D + first column of the lane) * 2.  Its stores then
// complete while the state update runs.
template <int NT>
__device__ __forceinline__ void rec_phase2(const ChunkImage &im, const RecRegs<NT> &R,
                                           __amdgpu_buffer_rsrc_t ro, int off_o, int rowb, int g,
                                           int j) {
  using TD = Tile<bf16_t, D>;
  using PL = PackedLower;
  constexpr int MB = NT == 1 ? 4 : 1;
#pragma unroll
  for (int m0 = 0; m0 < 4; m0 += MB) {
    bf16x8 qd[MB][4], mqk[MB][2];
#pragma unroll
    for (int mm = 0; mm < MB; ++mm) {
      const int m = m0 + mm;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) qd[mm][kb] = frag(im.Qd, TD::idx(16 * m + j, 32 * kb + 8 * g));
#pragma unroll
      for (int kb = 0; kb <= (m >> 1); ++kb) mqk[mm][kb] = frag(im.Mqk, PL::idx(16 * m + j, 32 * kb + 8 * g));
    }
#pragma unroll
    for (int mm = 0; mm < MB; ++mm)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int m = m0 + mm;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc = mfma_bf16_k32(R.sb[t][kb], qd[mm][kb], acc);
#pragma unroll
        for (int kb = 0; kb <= (m >> 1); ++kb) acc = mfma_bf16_k32(R.ub[t][kb], mqk[mm][kb], acc);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, to_bf16x4(acc)), ro,
                                              off_o + (16 * m) * rowb + 32 * t, 0, 0);
      }
  }
}

template <int NT>
__device__ __forceinline__ void rec_phase3(const ChunkImage &im, floatx4 (&S)[NT][8],
                                           const RecRegs<NT> &R, int g, int j) {
  using TC = Tile<bf16_t, CH>;
  constexpr int MS = NT == 1 ? 8 : 2;
#pragma unroll
  for (int m0 = 0; m0 < 8; m0 += MS) {
    bf16x8 krt[MS][2];
    float4 gam[MS];
#pragma unroll
    for (int mm = 0; mm < MS; ++mm) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) krt[mm][kb] = frag(im.KrT, TC::idx(16 * (m0 + mm) + j, 32 * kb + 8 * g));
      gam[mm] = *reinterpret_cast<const float4 *>(&im.gamC[16 * (m0 + mm) + 4 * g]);
    }
#pragma unroll
    for (int mm = 0; mm < MS; ++mm)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        floatx4 acc = S[t][m0 + mm];
        acc[0] *= gam[mm].x; acc[1] *= gam[mm].y; acc[2] *= gam[mm].z; acc[3] *= gam[mm].w;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) acc = mfma_bf16_k32(krt[mm][kb], R.ub[t][kb], acc);
        S[t][m0 + mm] = acc;
      }
  }
}

// The four phases back to back, from one image (the double-buffered kernel).
// with_o = false skips O (segment pairs, whose images are copied without
// Q_decay and M_qk).
template <int NT>
__device__ __forceinline__ void rec_step(const ChunkImage &im, floatx4 (&S)[NT][8], const bf16_t *V,
                                         int vld, int vcol, bool with_o, __amdgpu_buffer_rsrc_t ro,
                                         int off_o, int rowb, int g, int j) {
  RecRegs<NT> R;
  rec_phase0<NT>(im, S, V, vld, vcol, g, j, R);
  rec_phase1<NT>(im, g, j, R);
  if (with_o) rec_phase2<NT>(im, R, ro, off_o, rowb, g, j);
  rec_phase3<NT>(im, S, R, g, j);
}

// The chunk a slot holds: document d, its index k in the document, first token
// cs, len tokens (0: no chunk maps to the slot), whether it starts and whether
// it ends its document.
struct SlotChunk {
  int d;
  int64_t k;
  int64_t cs;
  int len;
  bool first, last;
};
__device__ __forceinline__ SlotChunk slot_chunk(const SplitParams &p, int64_t slot) {
  SlotChunk c;
  c.d = doc_of_slot(p.cu, p.N, slot);
  const int64_t a = uni64(cu_at(p.cu, p.T, c.d));
  const int64_t b = uni64(cu_at(p.cu, p.T, c.d + 1));
  c.k = slot - first_slot(a, c.d);
  c.cs = a + c.k * CH;
  c.len = c.cs < b ? (int)min((int64_t)CH, b - c.cs) : 0;
  c.first = c.cs == a;
  c.last = c.cs + c.len == b;
  return c;
}
// first slot in [s, s_end) that holds a chunk, or s_end
__device__ __forceinline__ int64_t next_chunk_slot(const SplitParams &p, int64_t s, int64_t s_end) {
  while (s < s_end && slot_chunk(p, s).len == 0) ++s;
  return s;
}

// L2 prefetch touches: one dword per L2 line (128 bytes) pulls the line in.
// Each touch holds one of the compute unit's outstanding L1 miss slots for a
// whole memory latency, the slots the copies need as well, so there is one per
// line and no more.  Parts of the image they cover: all operands, or for
// segment pairs only K_decay, K_restore^T, INV Diag(beta) and gamma^C.
constexpr int TOUCH_LINE = 128;
constexpr int IMG_LINES_ALL = (OFF_GAMC + 4 * D + TOUCH_LINE - 1) / TOUCH_LINE;
constexpr int KD_LINES = (OFF_QD - OFF_KD) / TOUCH_LINE;
constexpr int KRT_LINES = (OFF_MQK - OFF_KRT) / TOUCH_LINE;
constexpr int IMG_LINES_PAIRS = KD_LINES + KRT_LINES + (OFF_GAMC + 4 * D - OFF_INVB) / TOUCH_LINE;
static_assert(OFF_KD == 0 && OFF_GAMC == OFF_INVB + 2 * PackedLower::ELEMS, "image layout");
static_assert((OFF_QD - OFF_KD) % TOUCH_LINE == 0 && (OFF_MQK - OFF_KRT) % TOUCH_LINE == 0 &&
                  (OFF_GAMC + 4 * D - OFF_INVB) % TOUCH_LINE == 0 && OFF_INVB % TOUCH_LINE == 0,
              "touched parts must be whole lines");
__device__ __forceinline__ int touch_line_offset(int line, bool pairs_only) {
  if (!pairs_only) return TOUCH_LINE * line;
  if (line < KD_LINES) return TOUCH_LINE * line;
  if (line < KD_LINES + KRT_LINES) return OFF_KRT + TOUCH_LINE * (line - KD_LINES);
  return OFF_INVB + TOUCH_LINE * (line - KD_LINES - KRT_LINES);
}

// Items: documents (rmode 0), or segments of seg_slots chunk slots (rmode 1:
// re-run from the segment's entry state, writing O and the final states of
// documents ending inside; rmode 2: the segment's pair, state [S~ | M] from
// [0 | I] with v = 0 on the M columns).  At the first chunk of a document the
// state is reset to that document's initial state (M columns: 0), so a pair
// whose segment contains a document start has M = 0 and the scan needs no
// document logic.
template <int NT>
__global__ void __launch_bounds__(REC_THREADS, 1) kda_chunk_rec_kernel(SplitParams p) {
  using Smem = RecSmem<NT>;
  constexpr int SLICE = Smem::SLICE;
  constexpr int ES = 2;
  __shared__ Smem sm;

  const int nsplit = (p.rmode == 2 ? 4 : 2) / NT;
  const int units = (p.rmode == 0 ? p.N : p.n_seg) * p.H;
  const int xlo = blockIdx.x & 7;
  const int rest = blockIdx.x >> 3;
  const int split = rest % nsplit;
  const int unit = (rest / nsplit) * 8 + xlo;
  if (unit >= units) return;
  // documents in the order the prep wrote (longest first), else input order
  const int item = uni(p.rmode == 0 && p.order ? (int)cu_load(p.order, unit / p.H) : unit / p.H);
  const int h = unit % p.H;
  int64_t s_begin, s_end;
  if (p.rmode == 0) {
    const int64_t a = uni64(cu_at(p.cu, p.T, item));
    const int64_t b = uni64(cu_at(p.cu, p.T, item + 1));
    if (a == b) return;  // empty documents are handled by kda_copy_empty_kernel
    s_begin = first_slot(a, item);
    s_end = s_begin + (b - a + CH - 1) / CH;
  } else {
    s_begin = (int64_t)item * p.seg_slots;
    s_end = min(s_begin + p.seg_slots, p.n_slots);
  }
  s_begin = uni64(s_begin);
  s_end = uni64(s_end);
  const int col0 = split * SLICE;            // first state column of the workgroup
  const bool m_cols = col0 >= D;             // M columns of a pair: v = 0, start from I

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uni(tid >> 6);
  const bool copier = w >= REC_COMPUTE_WAVES;
  const int H = p.H;
  const int rowb = H * D * ES;

  if (copier) {
    // ---------------- copy waves ----------------
    const int cw = w - REC_COMPUTE_WAVES;                // 0 .. REC_COPY_WAVES - 1
    const int ct = tid - 64 * REC_COMPUTE_WAVES;         // 0 .. REC_COPY_THREADS - 1
    const bf16_t *v = (const bf16_t *)p.v;
    const char *img_h = (const char *)p.ws + (int64_t)h * p.n_slots * IMG_BYTES;
    const uint32_t lds_img = lds_addr(&sm.buf[0]);
    const uint32_t lds_v = lds_addr(&sm.V[0][0]);
    const uint32_t lds_sink = lds_addr(&sm.sink[0]);
    // v rows of a chunk, this workgroup's columns; rows past the chunk (and all
    // of them for M columns or past the range) read 0
    auto v_rsrc = [&](const SlotChunk &c, bool in_range) {
      const int bytes = (in_range && !m_cols && c.len > 0) ? ((c.len - 1) * H * D + SLICE) * ES : 0;
      return rsrc_words(v + (c.cs * H + h) * D + col0 % D, bytes);
    };
    // Pairs produce no O: Q_decay and M_qk are not copied.
    const bool pairs_only = p.rmode == 2;
    auto in_blocks = [](int blk, int lo, int hi) { return blk >= lo / 1024 && blk < hi / 1024; };
    // v rows in 1 KB blocks of VROWS token rows (LPR lanes per row)
    constexpr int LPR = SLICE * ES / 16;
    constexpr int VROWS = 64 / LPR;
    constexpr int VBLOCKS = CH / VROWS;
    // chunk of slot sl -> buffer kk & 1: v blocks cw, cw + REC_COPY_WAVES, ...,
    // the image in 1 KB blocks cw, cw + REC_COPY_WAVES, ...
    auto issue_copy = [&](int64_t sl, int kk) {
      const SlotChunk c = slot_chunk(p, sl);
      const i32x4 rv = v_rsrc(c, true);
      const uint32_t vdst = lds_v + (uint32_t)((kk & 1) * CH * SLICE * ES);
#pragma unroll
      for (int blk = cw; blk < VBLOCKS; blk += REC_COPY_WAVES) {
        copy16_to_lds(rv, vdst + blk * 1024, (VROWS * blk + lane / LPR) * rowb + (lane % LPR) * 16);
      }
      const i32x4 ri = rsrc_words(img_h + sl * IMG_BYTES, IMG_BYTES);
      const uint32_t dst = lds_img + (uint32_t)((kk & 1) * IMG_BYTES);
      for (int blk = cw; blk < IMG_BLOCKS; blk += REC_COPY_WAVES)
        if (!(pairs_only && (in_blocks(blk, OFF_QD, OFF_KRT) || in_blocks(blk, OFF_MQK, OFF_INVB))))
          copy16_to_lds(ri, dst + blk * 1024, lane * 16 + blk * 1024);
    };
    // L2 prefetch of slot sl: this workgroup's share of the image lines its
    // unit reads (one part per workgroup of the unit) and its v rows, one
    // dword per 64 bytes.  Always exactly TOUCH_OPS operations per wave
    // (offsets past the data, or a slot past the range, fetch nothing), so the
    // wait at the top of the loop can leave exactly these in flight.
    // (worst case: NT = 2 outside pair mode, one workgroup touches the whole image)
    constexpr int TOUCH_IMG = (NT == 1 ? (IMG_LINES_ALL + 1) / 2 : IMG_LINES_ALL) / REC_COPY_THREADS + 1;
    constexpr int TOUCH_OPS = TOUCH_IMG + 1;
    constexpr int OOB = 1 << 30;
    constexpr int VLINES = (SLICE * ES + TOUCH_LINE - 1) / TOUCH_LINE;  // lines per v row
    static_assert(CH * VLINES <= REC_COPY_THREADS, "v touch coverage");
    static_assert(TOUCH_IMG * REC_COPY_THREADS >= (NT == 1 ? (IMG_LINES_ALL + 1) / 2 : IMG_LINES_ALL),
                  "touch coverage");
    const int n_lines = pairs_only ? IMG_LINES_PAIRS : IMG_LINES_ALL;
    const int part_lines = (n_lines + nsplit - 1) / nsplit;
    auto issue_touch = [&](int64_t sl) {
      const bool in_range = sl < s_end;
      const SlotChunk c = slot_chunk(p, in_range ? sl : s_begin);
      const i32x4 ri = rsrc_words(img_h + sl * IMG_BYTES, in_range ? IMG_BYTES : 0);
#pragma unroll
      for (int i = 0; i < TOUCH_IMG; ++i) {
        const int k = i * REC_COPY_THREADS + ct;
        const int line = split * part_lines + k;
        touch4_to_lds(ri, lds_sink, k < part_lines && line < n_lines ? touch_line_offset(line, pairs_only) : OOB);
      }
      touch4_to_lds(v_rsrc(c, in_range), lds_sink,
                    ct < CH * VLINES ? (ct / VLINES) * rowb + (ct % VLINES) * TOUCH_LINE : OOB);
    };
    constexpr int AHEAD = 2;  // slots between a touch and the copy that uses it
    // The wait at the top of the loop leaves one touch batch in flight: one must
    // have been issued after every copy, the first included.
    static_assert(AHEAD >= 2, "a touch batch follows every copy");

    int64_t sl = next_chunk_slot(p, s_begin, s_end);
    if (sl < s_end) issue_copy(sl, 0);
    for (int i = 1; i < AHEAD; ++i) issue_touch(sl + i);
    for (int kk = 0; sl < s_end; ++kk) {
      const int64_t nsl = next_chunk_slot(p, sl + 1, s_end);
      // this wave's copy of the current chunk has landed (only the last touches
      // may still be in flight); after the barrier buffer (kk + 1) & 1 is free
      wait_vmem_except_last<TOUCH_OPS>();
      lds_barrier();
      if (nsl < s_end) issue_copy(nsl, kk + 1);
      issue_touch(sl + AHEAD);
      sl = nsl;
    }
    wait_vmem();  // no copy may still target this workgroup's LDS when it exits
    return;
  }

  // ---------------- compute waves ----------------
  const int g = lane >> 4;
  const int j = lane & 15;
  const int vcol = 16 * NT * w;  // first column of this wave within the slice
  const int colW = col0 + vcol;  // first state column of tile 0
  floatx4 S[NT][8];
  if (p.rmode == 1) {
    const float *e = uniptr(p.entry + ((int64_t)item * H + h) * (D * D));
#pragma unroll
    for (int t = 0; t < NT; ++t) state_load(S[t], e, D, colW + 16 * t, g, j);
    wait_vmem();  // before the loop: a wait inside it would also cover the O stores
  } else {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S[t][m][r] = (m_cols && 16 * m + 4 * g + r == colW + 16 * t + j - D) ? 1.f : 0.f;
  }
  bf16_t *o = (bf16_t *)p.o;
  const int off_o = (j * H * D + colW + 4 * g) * ES;  // token j, columns 4g..4g+3 of tile 0
  int64_t sl = next_chunk_slot(p, s_begin, s_end);
  for (int kk = 0; sl < s_end; ++kk) {
    const int64_t nsl = next_chunk_slot(p, sl + 1, s_end);
    const SlotChunk c = slot_chunk(p, sl);
    lds_barrier();  // the copy of this chunk is complete in buffer kk & 1
    if (c.first) {  // a document starts: its initial state (M columns: 0)
      if (!m_cols && p.init) {
        const float *s0 = uniptr(p.init + ((int64_t)c.d * H + h) * (D * D));
#pragma unroll
        for (int t = 0; t < NT; ++t) state_load(S[t], s0, D, colW + 16 * t, g, j);
        // Wait for these loads here.  Left to the compiler, the wait falls
        // where this branch rejoins the loop, on every chunk; with the previous
        // chunk's O stores pending on the same counter it must wait for those
        // too, and would hold every chunk until they had reached memory.
        wait_vmem();
      } else {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int m = 0; m < 8; ++m) S[t][m] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(o + (c.cs * H + h) * D, p.rmode != 2 ? ((c.len - 1) * H + 1) * D * ES : 0);
    if constexpr (NT == 1) {
      rec_step<NT>(sm.buf[kk & 1], S, &sm.V[kk & 1][0], SLICE, vcol, p.rmode != 2, ro, off_o, rowb, g, j);
    } else {
      // The per-lane operand addresses are cheap to form but would not all
      // fit in registers across the loop: derive them anew in each chunk from
      // a lane index the compiler cannot see through.
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int gi = ln >> 4, ji = ln & 15;
      rec_step<NT>(sm.buf[kk & 1], S, &sm.V[kk & 1][0], SLICE, vcol, p.rmode != 2, ro,
                   (ji * H * D + colW + 4 * gi) * ES, rowb, gi, ji);
    }
    if (c.last && p.rmode != 2 && p.final_state) {
      float *f = uniptr(p.final_state + ((int64_t)c.d * H + h) * (D * D));
#pragma unroll
      for (int t = 0; t < NT; ++t) state_store(S[t], f, D, colW + 16 * t, g, j);
    }
    // Checkpoints inside a document are ckpt_chunks or more slots apart (a later
    // document's first one lies ckpt_chunks - 1 slots past its first slot), so
    // slot / ckpt_chunks numbers them without collisions.
    if (p.ckpt_chunks > 0 && p.rmode != 2 && !c.last && (c.k + 1) % p.ckpt_chunks == 0) {
      float *f = uniptr(p.ckpt + ((sl / p.ckpt_chunks) * H + h) * (D * D));
#pragma unroll
      for (int t = 0; t < NT; ++t) state_store(S[t], f, D, colW + 16 * t, g, j);
    }
    sl = nsl;
  }
  if (p.rmode == 2) {  // the segment's pair [S~ | M]
    float *pr = uniptr(p.pairs + ((int64_t)item * H + h) * (D * 2 * D));
#pragma unroll
    for (int t = 0; t < NT; ++t) state_store(S[t], pr, 2 * D, colW + 16 * t, g, j);
  }
}

// ---------------------------------------------------------------------------
// The order in which the recurrence takes the documents.  Each (document,
// head) unit holds its workgroups for the document's whole chunk chain, and
// workgroups start in index order as compute units free up, so a long
// document that starts late ends late: with units in input order the step
// takes up to (total chunks / CUs) + longest chain, in longest-first order
// about the larger of the two.  Documents are sorted by decreasing chunk count
// rounded down to its leading 4 bits (a 256-bucket key, empty documents last);
// equal keys keep their input order, so the order is a fixed permutation of
// [0, N) whatever the timing.  One workgroup: a histogram pass, a scan of the
// buckets, and a placement pass that ranks equal keys with wave ballots.
// ---------------------------------------------------------------------------
constexpr int ORDER_THREADS = 256;
constexpr int ORDER_WAVES = ORDER_THREADS / 64;

// 0 for the most chunks ... 254 for one chunk; 255 for an empty document
__device__ __forceinline__ int order_key(const int32_t *cu, int d) {
  const int64_t a = cu[d], b = cu[d + 1];
  if (b <= a) return 255;
  const uint64_t c = (uint64_t)((b - a + CH - 1) / CH);
  const int e = 63 - __builtin_clzll(c);
  const int m = e >= 3 ? (int)((c >> (e - 3)) & 7) : (int)((c << (3 - e)) & 7);
  return 254 - min(8 * e + m, 254);
}

__global__ void __launch_bounds__(ORDER_THREADS) kda_doc_order_kernel(const int32_t *cu, int N,
                                                                        int32_t *order) {
  __shared__ int base[256];
  __shared__ int cnt[ORDER_WAVES][256];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  base[t] = 0;
  __syncthreads();
  for (int d = t; d < N; d += ORDER_THREADS) atomicAdd(&base[order_key(cu, d)], 1);
  __syncthreads();
  if (w == 0) {  // exclusive scan of the histogram, four buckets per lane
    int v[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = base[4 * lane + i]; s += v[i]; }
    int inc = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(inc, off);
      if (lane >= off) inc += o;
    }
    int run = inc - s;
#pragma unroll
    for (int i = 0; i < 4; ++i) { base[4 * lane + i] = run; run += v[i]; }
  }
  __syncthreads();
  for (int d0 = 0; d0 < N; d0 += ORDER_THREADS) {
#pragma unroll
    for (int i = 0; i < ORDER_WAVES; ++i) cnt[i][t] = 0;
    __syncthreads();
    const int d = d0 + t;
    const bool valid = d < N;
    const int k = valid ? order_key(cu, d) : 0;
    // lanes of this wave with the same key: the intersection over the key's
    // 8 bits of the lanes that agree on that bit
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool on = (k >> bit) & 1;
      const uint64_t ones = __ballot(valid && on);
      same &= on ? ones : ~ones;
    }
    const int rank = __popcll(same & ((1ull << lane) - 1));
    if (valid && rank == 0) cnt[w][k] = __popcll(same);
    __syncthreads();
    if (valid) {
      int pos = base[k] + rank;
      for (int i = 0; i < w; ++i) pos += cnt[i][k];
      order[pos] = d;
    }
    __syncthreads();
    int add = 0;
#pragma unroll
    for (int i = 0; i < ORDER_WAVES; ++i) add += cnt[i][t];
    base[t] += add;
    __syncthreads();
  }
}

hipError_t launch_chunk_prep(const SplitParams &p, hipStream_t stream) {
  if (p.order) {
    hipLaunchKernelGGL(kda_doc_order_kernel, dim3(1), dim3(ORDER_THREADS), 0, stream, p.cu, p.N,
                       p.order);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t blocks = p.n_slots * p.H;
  const dim3 grid((unsigned)blocks), block(FWD_THREADS);
  const bool unb = p.gate == GATE_SOFTPLUS;
  if (unb && p.raw)
    hipLaunchKernelGGL((kda_chunk_prep_kernel<true, true>), grid, block, 0, stream, p);
  else if (unb)
    hipLaunchKernelGGL((kda_chunk_prep_kernel<true, false>), grid, block, 0, stream, p);
  else if (p.raw)
    hipLaunchKernelGGL((kda_chunk_prep_kernel<false, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((kda_chunk_prep_kernel<false, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

// compute units of the current device (0 if unknown), cached per device
static int device_cus() {
  static int cached[64];
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64 && cached[dev] > 0) return cached[dev];
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) cached[dev] = cus;
  return cus;
}

hipError_t launch_chunk_recurrence(const SplitParams &p, hipStream_t stream) {
  // Two column tiles per compute wave once the workgroups that gives (one per
  // unit, two for a pair's 256 columns) fill the device; the workgroups of one
  // unit share an XCD
  const int units = (p.rmode == 0 ? p.N : p.n_seg) * p.H;
  const int cus = device_cus();
  const bool wide = units * (p.rmode == 2 ? 2 : 1) >= (cus > 0 ? cus : 256);
  const int groups = (units + 7) / 8;
  const int nsplit = (p.rmode == 2 ? 4 : 2) / (wide ? 2 : 1);
  const dim3 grid((unsigned)(groups * 8 * nsplit));
  if (wide)
    hipLaunchKernelGGL(kda_chunk_rec_kernel<2>, grid, dim3(REC_THREADS), 0, stream, p);
  else
    hipLaunchKernelGGL(kda_chunk_rec_kernel<1>, grid, dim3(REC_THREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kda
