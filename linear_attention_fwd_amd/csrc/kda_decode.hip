// kda_decode.hip -- fp32 decode step with speculative-verify replay (gfx950).
//
// One workgroup (4 waves) per (sequence, head).  The 128 x 128 fp32 state
// (64 KB) is streamed from HBM into VGPRs once, every replayed token (the
// accepted cached drafts, then the bonus token) is applied on chip, and the
// state is streamed back in place.  This is the design of the systems page
// ("Kimi K3 模型结构（7）", section "KDA：三种执行形态" on decode): cache only the
// projected inputs of the drafts and replay the accepted prefix, so the state
// crosses HBM once per step whatever the number of verified tokens.
//
// Per token the arithmetic is the delta form of the SemiAnalysis page
// (section "FlashKDA 算法"): S <- Diag(alpha) S; u = beta (v - S^T k);
// S <- S + k u^T; o = S^T q (output only for the bonus token).  About 7 D^2
// FLOP per token against 8 D^2 bytes of state traffic per step, so the kernel
// is bound by HBM bandwidth.
//
// Lane layout: wave w owns state columns [32w, 32w + 32).  Lane l holds
// columns 32w + 4(l % 8) .. +3 and rows 16(l / 8) .. +15, i.e. 64 floats.
// Column sums over the 128 rows reduce 16 rows in-lane, then across the 8
// row groups with three xor-shuffles; no barrier is needed between tokens.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int DEC_THREADS = 256;

// The drafts of the next window: inputs [N, W2, H, D] (beta [N, W2, H]) and
// their outputs o [N, W2, H, D]; W2 = 0 means none.
template <typename Tin> struct DecodeWindow {
  int W2;
  const Tin *q, *k, *v, *z, *beta;
  Tin *o;
};
constexpr int DEC_TOKBATCH = 8;  // tokens staged in LDS at a time
// bits of the error flag
constexpr int DEC_ERR_ACCEPTED = 1;  // an accepted length outside [0, W] was clamped
constexpr int DEC_ERR_SLOT = 2;      // a state slot outside [0, S_pool) was skipped


// RAW: q, k unnormalised and beta a logit (normalised and sigmoid applied here)
template <typename Tin, bool RAW>
__global__ void __launch_bounds__(DEC_THREADS)
kda_decode_kernel(float *__restrict__ state, const int32_t *__restrict__ slots,
                  const Tin *__restrict__ cq, const Tin *__restrict__ ck,
                  const Tin *__restrict__ cv, const Tin *__restrict__ cz,
                  const Tin *__restrict__ cbeta, const int32_t *__restrict__ accepted, int W,
                  const Tin *__restrict__ nq, const Tin *__restrict__ nk,
                  const Tin *__restrict__ nv, const Tin *__restrict__ nz,
                  const Tin *__restrict__ nbeta, DecodeWindow<Tin> win,
                  const float *__restrict__ A_log, float g_min, int gate, Tin *__restrict__ o,
                  int32_t *__restrict__ err_flag, int H, int S_pool) {
  __shared__ __align__(16) float s_k[DEC_TOKBATCH][D];
  __shared__ float s_qsc[DEC_TOKBATCH], s_ksc[DEC_TOKBATCH];  // raw inputs: 1 / ||q||, 1 / ||k||
  __shared__ __align__(16) float s_q[DEC_TOKBATCH][D];
  __shared__ __align__(16) float s_a[DEC_TOKBATCH][D];
  __shared__ __align__(16) float s_v[DEC_TOKBATCH][D];
  __shared__ float s_b[DEC_TOKBATCH];

  const int n = blockIdx.x / H;
  const int h = blockIdx.x % H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int cg = lane & 7;
  const int rg = lane >> 3;
  const int col0 = wave * 32 + cg * 4;
  const int row0 = rg * 16;

  // A slot outside the pool [0, S_pool) touches no state: the sequence's
  // outputs are written as zeros and DEC_ERR_SLOT is set in the error flag.
  const int64_t slot = slots ? (int64_t)slots[n] : (int64_t)n;
  if (slot < 0 || slot >= S_pool) {
    if (tid == 0 && err_flag)
      __hip_atomic_fetch_or(err_flag, DEC_ERR_SLOT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int x = tid; x < (1 + win.W2) * D; x += DEC_THREADS) {
      const int t = x / D, c = x % D;
      Tin *dst = t == 0 ? o + ((int64_t)n * H + h) * D
                        : win.o + (((int64_t)n * win.W2 + (t - 1)) * H + h) * D;
      io<Tin>::store1(dst + c, 0.f);
    }
    return;
  }
  int acc = accepted[n];
  if (acc < 0 || acc > W) {
    if (tid == 0 && err_flag)
      __hip_atomic_fetch_or(err_flag, DEC_ERR_ACCEPTED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    acc = acc < 0 ? 0 : W;
  }
  // tokens: the acc accepted drafts (replayed), the bonus token, then the
  // W2 drafts of the next window (outputs only; their states are not kept)
  const int ntok = acc + 1 + win.W2;
  float *__restrict__ Sg = state + (slot * H + h) * (int64_t)(D * D);

  // Stream the state slice into registers: 16 rows x 4 columns per lane.  The
  // state is touched once per step, so its loads and stores are non-temporal
  // (measured on a plain in-place stream of this size: 5.2 TB/s with ordinary
  // accesses, 5.4 TB/s with non-temporal ones).  Each wave keeps at most three
  // of its 16 loads (and later of its 16 stores) in flight: left to the
  // compiler, every wave issues all 16 at once, and the whole step ran at 5.33
  // TB/s of state traffic; with the loads and stores metered in pairs it runs
  // at 6.06 TB/s (at most one or two in flight: 5.98-6.01; at most eight:
  // 5.55; one at a time: 4.34).  With next-window drafts the kernel is no
  // longer a plain stream (their work follows the state stores) and runs
  // fastest unmetered: 1.20 ms, against 1.26 ms with either side metered.
  const bool meter = win.W2 == 0;
  float s[16][4];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const floatx4 x =
        __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(Sg + (row0 + i) * D + col0));
    s[i][0] = x[0]; s[i][1] = x[1]; s[i][2] = x[2]; s[i][3] = x[3];
    if ((i & 1) && i != 15 && meter) wait_vmem_except_last<1>();
  }

  const float escale = __expf(A_log ? A_log[h] : 0.0f);
  const float c1s = -escale * 1.4426950408889634f;  // unbounded gate, base 2

  for (int t0 = 0; t0 < ntok; t0 += DEC_TOKBATCH) {
    const int nb = min(DEC_TOKBATCH, ntok - t0);
    // Stage this batch of tokens: inputs converted to fp32, gate applied.
    for (int idx = tid; idx < nb * D; idx += DEC_THREADS) {
      const int tt = idx / D, c = idx % D;
      const int t = t0 + tt;
      const Tin *pq, *pk, *pv, *pz;
      if (t < acc) {
        const int64_t base = (((int64_t)n * W + t) * H + h) * D;
        pq = cq + base; pk = ck + base; pv = cv + base; pz = cz + base;
      } else if (t == acc) {
        const int64_t base = ((int64_t)n * H + h) * D;
        pq = nq + base; pk = nk + base; pv = nv + base; pz = nz + base;
      } else {
        const int64_t base = (((int64_t)n * win.W2 + (t - acc - 1)) * H + h) * D;
        pq = win.q + base; pk = win.k + base; pv = win.v + base; pz = win.z + base;
      }
      s_q[tt][c] = io<Tin>::load1(pq + c);
      s_k[tt][c] = io<Tin>::load1(pk + c);
      s_v[tt][c] = io<Tin>::load1(pv + c);
      const float zc = io<Tin>::load1(pz + c);
      s_a[tt][c] = gate == GATE_SOFTPLUS ? __builtin_amdgcn_exp2f(kda_gate2_softplus(zc, c1s))
                                         : __expf(kda_gate(zc, escale, g_min));
    }
    if (tid < nb) {
      const int t = t0 + tid;
      const float b = (t < acc)    ? io<Tin>::load1(cbeta + ((int64_t)n * W + t) * H + h)
                      : (t == acc) ? io<Tin>::load1(nbeta + (int64_t)n * H + h)
                                   : io<Tin>::load1(win.beta + ((int64_t)n * win.W2 + (t - acc - 1)) * H + h);
      s_b[tid] = RAW ? __builtin_amdgcn_rcpf(1.0f + __expf(-b)) : b;  // fp32, like the rest
    }
    __syncthreads();
    if constexpr (RAW) {  // L2 norms of q and k: wave w takes tokens w and w + 4 of the batch
      for (int tt = wave; tt < nb; tt += 4) {
        const float q0 = s_q[tt][lane], q1 = s_q[tt][lane + 64];
        const float k0 = s_k[tt][lane], k1 = s_k[tt][lane + 64];
        float sq = q0 * q0 + q1 * q1, sk = k0 * k0 + k1 * k1;
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
          sq += __shfl_xor(sq, m);
          sk += __shfl_xor(sk, m);
        }
        if (lane == 0) {
          s_qsc[tt] = sq > 0.f ? __builtin_amdgcn_rsqf(sq) : 0.f;
          s_ksc[tt] = sk > 0.f ? __builtin_amdgcn_rsqf(sk) : 0.f;
        }
      }
      __syncthreads();
    }

    // the last draft of a window is taken after the loop (no state update)
    const bool last_draft = win.W2 > 0 && t0 + nb == ntok;
    for (int tt = 0; tt < nb - (last_draft ? 1 : 0); ++tt) {
      const int t = t0 + tt;
      float kk[16], aa[16];
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        const float4 a4 = *reinterpret_cast<const float4 *>(&s_a[tt][row0 + i]);
        const float4 k4 = *reinterpret_cast<const float4 *>(&s_k[tt][row0 + i]);
        aa[i] = a4.x; aa[i + 1] = a4.y; aa[i + 2] = a4.z; aa[i + 3] = a4.w;
        kk[i] = k4.x; kk[i + 1] = k4.y; kk[i + 2] = k4.z; kk[i + 3] = k4.w;
      }
      if constexpr (RAW) {
        const float sc = s_ksc[tt];
#pragma unroll
        for (int i = 0; i < 16; ++i) kk[i] *= sc;
      }
      // decay, then the erase term against the decayed state
      float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          s[i][c] *= aa[i];
          p[c] = fmaf(s[i][c], kk[i], p[c]);
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        p[c] += __shfl_xor(p[c], 8);
        p[c] += __shfl_xor(p[c], 16);
        p[c] += __shfl_xor(p[c], 32);
      }
      const float4 v4 = *reinterpret_cast<const float4 *>(&s_v[tt][col0]);
      const float bt = s_b[tt];
      float u[4];
      u[0] = bt * (v4.x - p[0]);
      u[1] = bt * (v4.y - p[1]);
      u[2] = bt * (v4.z - p[2]);
      u[3] = bt * (v4.w - p[3]);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
#pragma unroll
        for (int c = 0; c < 4; ++c) s[i][c] = fmaf(kk[i], u[c], s[i][c]);
      }
      if (t >= acc) {  // the bonus token and the next window: o = S^T q
        float qq[16], ob[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
          const float4 q4 = *reinterpret_cast<const float4 *>(&s_q[tt][row0 + i]);
          qq[i] = q4.x; qq[i + 1] = q4.y; qq[i + 2] = q4.z; qq[i + 3] = q4.w;
        }
        if constexpr (RAW) {
          const float sc = s_qsc[tt];
#pragma unroll
          for (int i = 0; i < 16; ++i) qq[i] *= sc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
#pragma unroll
          for (int c = 0; c < 4; ++c) ob[c] = fmaf(s[i][c], qq[i], ob[c]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          ob[c] += __shfl_xor(ob[c], 8);
          ob[c] += __shfl_xor(ob[c], 16);
          ob[c] += __shfl_xor(ob[c], 32);
        }
        if (rg == 0) {
          Tin *dst = (t == acc) ? o + ((int64_t)n * H + h) * D
                                : win.o + (((int64_t)n * win.W2 + (t - acc - 1)) * H + h) * D;
          io<Tin>::store4(dst + col0, ob);
        }
      }
      if (t == acc) {  // the state after the bonus token is the one kept
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_nontemporal_store(floatx4{s[i][0], s[i][1], s[i][2], s[i][3]},
                                      reinterpret_cast<floatx4 *>(Sg + (row0 + i) * D + col0));
          if ((i & 1) && i != 15 && meter) wait_vmem_except_last<1>();  // as the loads
        }
      }
    }
    if (last_draft) {
      // The last draft of the window: its state is not kept, so the update is
      // not formed.  With S' = Diag(alpha) S and u = beta (v - S^T k), its
      // output (S' + k u^T)^T q = S^T (alpha q) + (k^T q) u needs one pass over
      // S (two weighted column sums) instead of decay, erase, update and read.
      const int tt = nb - 1;
      const int t = t0 + tt;
      const float qsc = RAW ? s_qsc[tt] : 1.f, ksc = RAW ? s_ksc[tt] : 1.f;
      float p[4] = {0.f, 0.f, 0.f, 0.f}, ob[4] = {0.f, 0.f, 0.f, 0.f}, kq = 0.f;
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        const float4 a4 = *reinterpret_cast<const float4 *>(&s_a[tt][row0 + i]);
        const float4 k4 = *reinterpret_cast<const float4 *>(&s_k[tt][row0 + i]);
        const float4 q4 = *reinterpret_cast<const float4 *>(&s_q[tt][row0 + i]);
        const float av[4] = {a4.x, a4.y, a4.z, a4.w};
        const float kv[4] = {k4.x * ksc, k4.y * ksc, k4.z * ksc, k4.w * ksc};
        const float qv[4] = {q4.x * qsc, q4.y * qsc, q4.z * qsc, q4.w * qsc};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ak = av[r] * kv[r], aq = av[r] * qv[r];
          kq = fmaf(kv[r], qv[r], kq);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            p[c] = fmaf(s[i + r][c], ak, p[c]);
            ob[c] = fmaf(s[i + r][c], aq, ob[c]);
          }
        }
      }
#pragma unroll
      for (int m = 8; m < 64; m <<= 1) {
        kq += __shfl_xor(kq, m);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          p[c] += __shfl_xor(p[c], m);
          ob[c] += __shfl_xor(ob[c], m);
        }
      }
      if (rg == 0) {
        const float4 v4 = *reinterpret_cast<const float4 *>(&s_v[tt][col0]);
        const float bt = s_b[tt];
        const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) ob[c] = fmaf(kq, bt * (vv[c] - p[c]), ob[c]);
        io<Tin>::store4(win.o + (((int64_t)n * win.W2 + (t - acc - 1)) * H + h) * D + col0, ob);
      }
    }
    __syncthreads();  // the staging buffers are rewritten by the next batch
  }
}

template <typename Tin>
hipError_t launch_decode(float *state, const int32_t *slots, const void *cq, const void *ck,
                         const void *cv, const void *cz, const void *cbeta,
                         const int32_t *accepted, int W, const void *nq, const void *nk,
                         const void *nv, const void *nz, const void *nbeta,
                         const DecodeWindowArgs &w, bool raw, const float *A_log, float g_min,
                         int gate, void *o, int32_t *err_flag, int N, int H, int S_pool,
                         hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)N * H));
  DecodeWindow<Tin> win{w.W2, (const Tin *)w.q, (const Tin *)w.k, (const Tin *)w.v,
                        (const Tin *)w.z, (const Tin *)w.beta, (Tin *)w.o};
  auto kernel = raw ? kda_decode_kernel<Tin, true> : kda_decode_kernel<Tin, false>;
  hipLaunchKernelGGL(kernel, grid, dim3(DEC_THREADS), 0, stream, state, slots, (const Tin *)cq,
                     (const Tin *)ck, (const Tin *)cv, (const Tin *)cz, (const Tin *)cbeta,
                     accepted, W, (const Tin *)nq, (const Tin *)nk, (const Tin *)nv,
                     (const Tin *)nz, (const Tin *)nbeta, win, A_log, g_min, gate, (Tin *)o, err_flag,
                     H, S_pool);
  return hipGetLastError();
}

template hipError_t launch_decode<float>(float *, const int32_t *, const void *, const void *,
                                         const void *, const void *, const void *,
                                         const int32_t *, int, const void *, const void *,
                                         const void *, const void *, const void *,
                                         const DecodeWindowArgs &, bool, const float *, float,
                                         int, void *, int32_t *, int, int, int, hipStream_t);
template hipError_t launch_decode<bf16_t>(float *, const int32_t *, const void *, const void *,
                                          const void *, const void *, const void *,
                                          const int32_t *, int, const void *, const void *,
                                          const void *, const void *, const void *,
                                          const DecodeWindowArgs &, bool, const float *, float,
                                          int, void *, int32_t *, int, int, int, hipStream_t);

}  // namespace kda
