// kda_split.hip -- two-kernel chunkwise KDA prefill for gfx950 (bf16 operands).
//
// The chunk prep (stages a1-a4 of kda_chunk.h) depends only on the chunk's own
// tokens, so it runs token-parallel over every (head, chunk) at once: one
// workgroup per chunk, two workgroups per compute unit.  It writes the
// recurrence operands of its chunk, the "chunk image", to a workspace in the
// exact layout of the recurrence kernel's LDS tiles.  The recurrence kernel
// then runs the serial chain of each (document, head, 64-column slice) and only
// streams images: global -> LDS copies into a double buffer, one chunk ahead
// of the MFMA work (the split into a prep kernel and a recurrence kernel is the
// FlashKDA structure of the SemiAnalysis page, section "FlashKDA 算法").
//
// Chunks restart at every document start; chunk k of document d has slot
// first_slot(d) + k (kda_launch.h), the images of head h lie at
// ws + (h * n_slots + slot) * sizeof(ChunkImage).
#include <stddef.h>

#include "kda_chunk.h"

namespace kda {

// Recurrence operands of one (head, chunk), laid out as LDS tiles.
struct __align__(16) ChunkImage {
  bf16_t Kd[CH * D];     // K_decay, channel axis permuted
  bf16_t Qd[CH * D];     // Q_decay, channel axis permuted
  bf16_t KrT[D * CH];    // K_restore^T, token axis permuted
  bf16_t Mqk[CH * CH];   // M_qk, token axis permuted
  bf16_t INVb[CH * CH];  // INV Diag(beta), token axis permuted
  float gamC[D];         // gamma^C
  float pad[D];          // the image is a whole number of 1 KB copy blocks
};
constexpr int IMG_BYTES = (int)sizeof(ChunkImage);
constexpr int IMG_BLOCKS = IMG_BYTES / 1024;
static_assert(IMG_BYTES % 1024 == 0, "chunk image must be whole 1 KB blocks");
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
struct __align__(16) PrepSmem {
  union {
    struct {
      bf16_t Qh[CH * D];  // q_i e^(G_i - G_s(i))
      bf16_t Kh[CH * D];  // k_i e^(G_i - G_s(i))
      bf16_t Ki[CH * D];  // k_j e^(G_s(j) - G_j)
    } p1;
    bf16_t INVb[CH * CH];  // staged after the subtile operands are dead
  } u;
  float L[CH * CH];
  bf16_t Tdg[4][SUB * SUB];
  PrepLds ps;
};

__global__ void __launch_bounds__(FWD_THREADS, 2) kda_chunk_prep_kernel(SplitParams p) {
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

  float G[4][8];
  prep_gate_cumsum<IO>(sm.ps, Rz, Rb, c1, gmin2, len, tid, w, tq, cg, G);  // two barriers

  const __amdgpu_buffer_rsrc_t ri =
      make_rsrc((char *)p.ws + ((int64_t)h * p.n_slots + slot) * IMG_BYTES, IMG_BYTES);
  float Kres[4][8];
  prep_decay_operands<Ar, IO>(sm.ps, sm.u.p1.Qh, sm.u.p1.Kh, sm.u.p1.Ki, Rq, Rk, G, w, tq, cg, Kres,
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
  prep_pair_factors(sm.ps, tid);
  if (tid < D) buf_st_f32(ri, __builtin_amdgcn_exp2f(sm.ps.GC2[tid]), OFF_GAMC + 4 * tid);
  __syncthreads();
  SCHED_FENCE();

  prep_subtile_products<Ar>(sm.ps, sm.u.p1.Qh, sm.u.p1.Kh, sm.u.p1.Ki, sm.L, w, g, j,
                            [&](int row, int J, const float *mq) {
                              img_st4(ri, OFF_MQK + 2 * TC::idx(row, kperm(16 * J + 4 * g)), mq);
                            });
  // The recurrence reads the upper blocks (0,1) and (2,3) of M_qk and INV Diag(beta)
  // (its 32-wide k steps span two subtiles); they must hold zeros.
  const float zero4[4] = {0.f, 0.f, 0.f, 0.f};
  if (w & 1) img_st4(ri, OFF_MQK + 2 * TC::idx(16 * (w - 1) + j, kperm(16 * w + 4 * g)), zero4);
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
  // INV Diag(beta): staged tile -> image, 16 bytes per lane
  for (int x = tid; x < CH * CH * 2 / 16; x += FWD_THREADS) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(sm.u.INVb) + 16 * x);
    __builtin_amdgcn_raw_buffer_store_b128(v, ri, OFF_INVB + 16 * x, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Recurrence: one workgroup per (document, head, 64-column slice); slices of
// one (document, head) share an XCD (blockIdx % 8), so the second reads the
// images from L2.
// ---------------------------------------------------------------------------
struct __align__(16) RecSmem {
  ChunkImage buf[2];
};

// MFMA A-operand fragments of one chunk for one wave, read from the chunk image
// in LDS ahead of use.  None depends on the state, so the reads of the state
// path (K_decay, INV, K_restore^T, gamma) are all in flight before the chunk's
// first product and the chain then runs without waiting on LDS; the output
// operands (Q_decay, M_qk) are read once the first products are issued, into
// registers the K_decay fragments free.  Lane (g, j) holds row 16m + j,
// k elements 32kb + 8g .. +7 of each tile (the k32 operand layout).
struct StateFrags {
  bf16x8 kd[4][4];   // K_decay   [m][kb]
  bf16x8 inv[6];     // INV Diag(beta), blocks (m, kb <= m/2) in m-major order
  bf16x8 krt[8][2];  // K_restore^T [m][kb]
  float4 gam[8];     // gamma^C rows 16m + 4g .. +3
};
struct OutFrags {
  bf16x8 qd[4][4];   // Q_decay   [m][kb]
  bf16x8 mqk[6];     // M_qk, as inv
};

__device__ __forceinline__ bf16x8 frag(const bf16_t *tile, int idx) {
  return *reinterpret_cast<const bf16x8 *>(tile + idx);
}
__device__ __forceinline__ void load_state_frags(StateFrags &f, const ChunkImage &im, int g, int j) {
  using TD = Tile<bf16_t, D>;
  using TC = Tile<bf16_t, CH>;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) f.kd[m][kb] = frag(im.Kd, TD::idx(16 * m + j, 32 * kb + 8 * g));
  int x = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int kb = 0; kb <= (m >> 1); ++kb, ++x) f.inv[x] = frag(im.INVb, TC::idx(16 * m + j, 32 * kb + 8 * g));
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) f.krt[m][kb] = frag(im.KrT, TC::idx(16 * m + j, 32 * kb + 8 * g));
#pragma unroll
  for (int m = 0; m < 8; ++m) f.gam[m] = *reinterpret_cast<const float4 *>(&im.gamC[16 * m + 4 * g]);
}
__device__ __forceinline__ void load_out_frags(OutFrags &f, const ChunkImage &im, int g, int j) {
  using TD = Tile<bf16_t, D>;
  using TC = Tile<bf16_t, CH>;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) f.qd[m][kb] = frag(im.Qd, TD::idx(16 * m + j, 32 * kb + 8 * g));
  int x = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int kb = 0; kb <= (m >> 1); ++kb, ++x) f.mqk[x] = frag(im.Mqk, TC::idx(16 * m + j, 32 * kb + 8 * g));
}

__device__ __forceinline__ bf16x8 pack_tiles(floatx4 t0, floatx4 t1) {
  return to_bf16x8(floatx8{t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]});
}

// The chunk recurrence (chunk_recurrence in kda_chunk.h) on staged fragments:
//   U = INV Diag(beta) (V - K_decay S);  O = Q_decay S + M_qk U;
//   S <- Diag(gamma^C) S + K_restore^T U.
__device__ __forceinline__ void rec_step(const ChunkImage &im, floatx4 (&S)[8], const floatx4 (&Vt)[4],
                                         __amdgpu_buffer_rsrc_t ro, int off_v, int rowb, int g,
                                         int j) {
  using IO = bufio<bf16_t>;
  StateFrags f;
  load_state_frags(f, im, g, j);
  bf16x8 sb[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) sb[kb] = pack_tiles(S[2 * kb], S[2 * kb + 1]);
  floatx4 U[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    floatx4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) x = mfma_bf16_k32(f.kd[m][kb], sb[kb], x);
    U[m] = Vt[m] - x;
  }
  SCHED_FENCE();
  OutFrags fo;
  load_out_frags(fo, im, g, j);
  bf16x8 bb[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) bb[kb] = pack_tiles(U[2 * kb], U[2 * kb + 1]);
  int x = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb <= (m >> 1); ++kb, ++x) acc = mfma_bf16_k32(f.inv[x], bb[kb], acc);
    U[m] = acc;
  }
  bf16x8 ub[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) ub[kb] = pack_tiles(U[2 * kb], U[2 * kb + 1]);
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    floatx4 acc = S[m];
    acc[0] *= f.gam[m].x; acc[1] *= f.gam[m].y; acc[2] *= f.gam[m].z; acc[3] *= f.gam[m].w;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) acc = mfma_bf16_k32(f.krt[m][kb], ub[kb], acc);
    S[m] = acc;
  }
  x = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) acc = mfma_bf16_k32(fo.qd[m][kb], sb[kb], acc);
#pragma unroll
    for (int kb = 0; kb <= (m >> 1); ++kb, ++x) acc = mfma_bf16_k32(fo.mqk[x], ub[kb], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) IO::st1(ro, acc[r], off_v + (16 * m + r) * rowb);
  }
}

__global__ void __launch_bounds__(FWD_THREADS, 1) kda_chunk_rec_kernel(SplitParams p) {
  using IO = bufio<bf16_t>;
  constexpr int ES = 2;
  __shared__ RecSmem sm;

  const int units = p.N * p.H;
  const int xlo = blockIdx.x & 7;
  const int rest = blockIdx.x >> 3;
  const int split = rest & 1;
  const int unit = (rest >> 1) * 8 + xlo;
  if (unit >= units) return;
  const int d = unit / p.H;
  const int h = unit % p.H;
  const int64_t a = uni64(cu_at(p.cu, p.T, d));
  const int64_t b = uni64(cu_at(p.cu, p.T, d + 1));
  if (a == b) return;  // empty documents are handled by kda_copy_empty_kernel

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uni(tid >> 6);
  const int g = lane >> 4;
  const int j = lane & 15;
  const int colW = split * 64 + w * 16;
  const int H = p.H;

  floatx4 S[8];
  if (p.init) {
    state_load(S, uniptr(p.init + ((int64_t)d * H + h) * (D * D)), D, colW, g, j);
  } else {
#pragma unroll
    for (int m = 0; m < 8; ++m) S[m] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  const bf16_t *v = (const bf16_t *)p.v;
  bf16_t *o = (bf16_t *)p.o;
  const int rowb = H * D * ES;
  const int off_v = (4 * g * H * D + colW + j) * ES;
  const int nch = (int)((b - a + CH - 1) / CH);
  const char *img0 = (const char *)p.ws + ((int64_t)h * p.n_slots + first_slot(a, d)) * IMG_BYTES;
  const uint32_t lds0 = lds_addr(&sm.buf[0]);

  // image of chunk kk -> buffer kk & 1, 1 KB blocks dealt round-robin to the waves
  auto issue_image = [&](int kk) {
    const i32x4 rs = rsrc_words(img0 + (int64_t)kk * IMG_BYTES, IMG_BYTES);
    const uint32_t dst = lds0 + (uint32_t)((kk & 1) * IMG_BYTES);
    for (int blk = w; blk < IMG_BLOCKS; blk += 4) copy16_to_lds(rs, dst + blk * 1024, lane * 16 + blk * 1024);
  };
  typename IO::raw1 Rv[4][4];
  auto fetch_v = [&](int kk) {
    const int64_t c0 = a + (int64_t)kk * CH;
    const int n = (int)min((int64_t)CH, b - c0);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + (c0 * H + h) * D, ((n - 1) * H + 1) * D * ES);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) Rv[m][r] = IO::ld1(rv, off_v + (16 * m + r) * rowb);
  };

  issue_image(0);
  fetch_v(0);
  for (int kk = 0; kk < nch; ++kk) {
    const int64_t cs = a + (int64_t)kk * CH;
    const int len = (int)min((int64_t)CH, b - cs);
    wait_vmem();      // this wave's copies of image kk (and V of chunk kk) have landed
    __syncthreads();  // ... and every wave's; buffer (kk + 1) & 1 is no longer read
    floatx4 Vt[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) Vt[m][r] = IO::cvt1(Rv[m][r]);
    if (kk + 1 < nch) {
      issue_image(kk + 1);
      fetch_v(kk + 1);
    }
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(o + (cs * H + h) * D, ((len - 1) * H + 1) * D * ES);
    rec_step(sm.buf[kk & 1], S, Vt, ro, off_v, rowb, g, j);
  }
  if (p.final_state) state_store(S, uniptr(p.final_state + ((int64_t)d * H + h) * (D * D)), D, colW, g, j);
}

size_t split_workspace_bytes(int64_t T, int N, int H) {
  return (size_t)n_chunk_slots(T, N) * (size_t)H * (size_t)IMG_BYTES;
}

hipError_t launch_chunk_prep(const SplitParams &p, hipStream_t stream) {
  const int64_t blocks = p.n_slots * p.H;
  hipLaunchKernelGGL(kda_chunk_prep_kernel, dim3((unsigned)blocks), dim3(FWD_THREADS), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_chunk_recurrence(const SplitParams &p, hipStream_t stream) {
  const int units = p.N * p.H;
  const int groups = (units + 7) / 8;
  hipLaunchKernelGGL(kda_chunk_rec_kernel, dim3((unsigned)(groups * 8 * 2)), dim3(FWD_THREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kda
