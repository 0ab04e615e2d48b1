// kda_scan.hip -- scan of segment pairs into exact entry states (gfx950).
//
// Equation (17) of "Kimi K3 模型结构（7）：结构决定系统" and steps 2-4 of its
// derivation: a segment maps its entry state E to M E + S~, and the entry
// state of segment j+1 is E_{j+1} = M_j E_j + S~_j.  Where a document starts
// exactly on the boundary of segment j the state is reset to that document's
// own initial state instead (section "文档边界"); documents starting strictly
// inside a segment are folded into that segment's pair (M = 0) upstream.
//
// One workgroup per (head, 16-column slice of the state); columns of E never
// mix in E <- M E + S~, so slices are independent.  Each of the 4 waves owns
// 32 rows of E; the current E slice is shared through LDS (transposed so a
// lane's B operand is one contiguous read, double-buffered so one barrier per
// step suffices).  The scan is serial over segments, so each step's pair is
// loaded during the previous step.  This one-level scan serves the fp32
// arithmetic path (fp32 MFMA); the bf16 path scans its pairs in three levels
// with kda_scan_chains_kernel below, whose products use a hi/lo bf16 split of
// both operands (three MFMAs, about 16 mantissa bits), since errors in M E
// would otherwise propagate along the whole scan.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int SCAN_THREADS = 256;

// Workgroups are dispatched to the 8 XCDs round-robin by block index, and every
// XCD has its own L2.  All column slices of one unit (a head, or a chain and
// head) read the same M rows, so they are given block indices congruent mod 8:
// block b serves slice (b / 8) % nslices of unit (b / (8 nslices)) * 8 + b % 8.
// The grid is rounded up to whole groups of 8 units; blocks past the last unit
// exit at once.
struct ScanBlock {
  int unit, slice;
};
__device__ __forceinline__ ScanBlock scan_block(int nslices) {
  const int b = blockIdx.x;
  const int q = b >> 3;
  return ScanBlock{(q / nslices) * 8 + (b & 7), q % nslices};
}
inline unsigned scan_grid(int64_t units, int nslices) {
  return (unsigned)((units + 7) / 8 * 8 * nslices);
}

__device__ __forceinline__ int scan_doc_of(const int32_t *cu, int N, int64_t pos) {
  if (!cu) return 0;
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= pos) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The operands of one scan step for this lane: rows 32w + 16t + j of M (the
// A operand, 8 consecutive columns per k block) and S~ at rows 32w + 16t + 4g
// + r, column col.  They do not depend on E, so the next step's are loaded
// while the current step computes.
struct ScanOps {
  float4 m[2][4][2];  // [t][kb][half]
  floatx4 st[2];
};

__global__ void __launch_bounds__(SCAN_THREADS, 1)
kda_pair_scan_kernel(const float *__restrict__ pairs, const float *__restrict__ S0,
                     const int32_t *__restrict__ cu, int N, int H, int n_seg, int64_t seg_len,
                     float *__restrict__ entry) {
  __shared__ __align__(16) float ET[2][16][D];  // E slice, [buffer][column][row]

  const ScanBlock sb = scan_block(8);
  if (sb.unit >= H) return;
  const int h = sb.unit;
  const int cs = sb.slice;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int g = lane >> 4;
  const int j = lane & 15;
  const int col = 16 * cs + j;

  auto row_of = [&](int t, int r) { return 32 * w + 16 * t + 4 * g + r; };
  auto load_state = [&](const float *src, floatx4 (&E)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) E[t][r] = src ? src[row_of(t, r) * D + col] : 0.f;
  };
  auto publish = [&](int seg, const floatx4 (&E)[2]) {
    float *dst = entry + ((int64_t)seg * H + h) * (D * D);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        dst[row_of(t, r) * D + col] = E[t][r];
        ET[seg & 1][j][row_of(t, r)] = E[t][r];
      }
  };
  auto doc_state = [&](int d) -> const float * {
    return S0 ? S0 + ((int64_t)d * H + h) * (D * D) : nullptr;
  };
  // operands of the step producing E_s from segment s - 1's pair
  auto load_ops = [&](int s, ScanOps &o) {
    const float *P = pairs + ((int64_t)(s - 1) * H + h) * (D * 2 * D);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) o.st[t][r] = P[row_of(t, r) * (2 * D) + col];  // S~
      const float *Mrow = P + (32 * w + 16 * t + j) * (2 * D) + D;             // row of M
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        o.m[t][kb][0] = *reinterpret_cast<const float4 *>(Mrow + 32 * kb + 8 * g);
        o.m[t][kb][1] = *reinterpret_cast<const float4 *>(Mrow + 32 * kb + 8 * g + 4);
      }
    }
  };
  // E_s = M E_{s-1} + S~ (E_{s-1} read from ET[(s - 1) & 1])
  auto step = [&](int s, const ScanOps &o, floatx4 (&E)[2]) {
    const int pb = (s - 1) & 1;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      floatx4 acc = o.st[t];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float4 a0 = o.m[t][kb][0], a1 = o.m[t][kb][1];
        const float4 b0 = *reinterpret_cast<const float4 *>(&ET[pb][j][32 * kb + 8 * g]);
        const float4 b1 = *reinterpret_cast<const float4 *>(&ET[pb][j][32 * kb + 8 * g + 4]);
        const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = mfma_f32_k4(av[e], bv[e], acc);
      }
      E[t] = acc;
    }
  };

  floatx4 E[2];
  load_state(doc_state(scan_doc_of(cu, N, 0)), E);
  publish(0, E);
  ScanOps ops[2];
  if (n_seg > 1) load_ops(1, ops[1]);
  __syncthreads();

  // Segment s's entry state from the previous one; the operands of step s + 1
  // load while step s computes (two register sets, alternating).  One barrier
  // per step: E_s is written to the other LDS buffer than E_{s-1}.
  // (The prefetch is unconditional -- the last step reloads its own operands --
  // so that the compiler's wait counts never have to cover a path without it.)
  auto body = [&](int s, ScanOps &cur, ScanOps &nxt) {
    load_ops(min(s + 1, n_seg - 1), nxt);
    const int64_t pos = (int64_t)s * seg_len;
    const int d = scan_doc_of(cu, N, pos);
    const bool reset = cu ? ((int64_t)cu[d] == pos) : false;
    if (reset) {
      load_state(doc_state(d), E);
    } else {
      step(s, cur, E);
    }
    publish(s, E);
    lds_barrier();  // LDS only: the next step's operand loads stay in flight
  };
  int s = 1;
  for (; s + 1 < n_seg; s += 2) {
    body(s, ops[1], ops[0]);
    body(s + 1, ops[0], ops[1]);
  }
  if (s < n_seg) body(s, ops[1], ops[0]);
}

// ---------------------------------------------------------------------------
// Chains of pair applications, for a scan of segment pairs in levels.  A chain
// walks pairs first..last (last exclusive) of the pair array and keeps a state
// X with ncols columns:
//   mode 0 (states): X starts from init[chain] (or 0) and the state before each
//     pair, X_i, is written to states[i]; X <- M_i X + S~_i; with write_final
//     the state after the chain's last pair is written too, to states[last]
//     (a chain of no pairs then writes its start state);
//   mode 1 (compose): X = [S~ | M] of the first pair, then X <- M_i X + [S~_i | 0]
//     for the others, i.e. the pairs composed into one; written to composed[chain].
// One workgroup per (chain, head, slice of 16 CT columns of X) with 8 / RT
// waves; wave w owns rows 16 RT w .. 16 RT (w + 1) - 1 and every 16-column
// tile of the slice, so every M row it loads (and splits into bf16 halves)
// serves CT tiles.  Same step as the pair scan: M rows as the A operand from
// the pair array (the next step's loaded during the current one), the X slice
// from LDS (double-buffered, split into bf16 halves once by its owner),
// products in bf16 hi/lo halves (three MFMAs per k block and tile).
// ---------------------------------------------------------------------------
template <int CT, int RT> struct ChainOps {
  float4 m[RT][4][2];  // [row tile][kb][half]: M rows 16 RT w + 16 t + j
  floatx4 st[CT][RT];  // [column tile][row tile]: S~ (0 on M columns, read out of bounds)
};

template <int CT, int RT>
__global__ void __launch_bounds__(512 / RT) kda_scan_chains_kernel(ScanChains sc) {
  constexpr int COLS = 16 * CT;
  constexpr int ROWS = 16 * RT;  // rows per wave
  using Ops = ChainOps<CT, RT>;
  // X slice split into bf16 high and low halves by the wave that owns each
  // value, so the B operands are read ready-made: [buffer][column][row]
  __shared__ __align__(16) bf16_t XH[2][COLS][D];
  __shared__ __align__(16) bf16_t XL[2][COLS][D];

  const int nslices = sc.ncols / COLS;
  const ScanBlock sb = scan_block(nslices);
  if (sb.unit >= sc.n_chains * sc.H) return;
  const int chain = sb.unit / sc.H;
  const int h = sb.unit % sc.H;
  const int c0 = COLS * sb.slice;  // first column of the slice (S~ part below D, M part from D on)
  const int first = chain * sc.chain_len;
  const int last = min(first + sc.chain_len, sc.n_pairs);
  const bool final_write = sc.mode == 0 && sc.write_final;
  if (first >= last && !final_write) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int g = lane >> 4;
  const int j = lane & 15;
  const bool st_on = c0 < D;  // the slice lies in the S~ columns (D is a multiple of the slice)

  auto row_of = [&](int t, int r) { return ROWS * w + 16 * t + 4 * g + r; };
  auto col_of = [&](int c) { return c0 + 16 * c + j; };
  auto pair_at = [&](int i) { return sc.pairs + ((int64_t)i * sc.H + h) * (D * 2 * D); };
  auto share = [&](int buf, const floatx4 (&X)[CT][RT]) {
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        bf16x4 hi, lo;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          hi[r] = (__bf16)X[c][t][r];
          lo[r] = (__bf16)(X[c][t][r] - (float)hi[r]);
        }
        *reinterpret_cast<bf16x4 *>(&XH[buf][16 * c + j][row_of(t, 0)]) = hi;
        *reinterpret_cast<bf16x4 *>(&XL[buf][16 * c + j][row_of(t, 0)]) = lo;
      }
  };
  // Global accesses go through buffer descriptors: one per-lane offset, with
  // the per-element constants in the scalar offset, so that no array of
  // per-element addresses has to stay live across the loop.
  auto write_state = [&](float *dst, int ld, const floatx4 (&X)[CT][RT]) {
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dst, D * ld * 4);
    const int voff = ((ROWS * w + 4 * g) * ld + c0 + j) * 4;
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(X[c][t][r]), rd, voff,
                                                ((16 * t + r) * ld + 16 * c) * 4, 0);
  };
  auto load_ops = [&](int i, Ops &o) {
    const float *P = pair_at(i);
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(P, D * 2 * D * 4);
    // S~ through a descriptor of size 0 on the M columns: those loads return 0
    // and move no data
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(P, st_on ? D * 2 * D * 4 : 0);
    const int voff_st = ((ROWS * w + 4 * g) * (2 * D) + (c0 & (D - 1)) + j) * 4;
    const int voff_m = ((ROWS * w + j) * (2 * D) + D + 8 * g) * 4;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          o.st[c][t][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
              rs, voff_st, ((16 * t + r) * (2 * D) + 16 * c) * 4, 0));
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(
              rp, voff_m, (16 * t * (2 * D) + 32 * kb + 4 * hf) * 4, 0);
          o.m[t][kb][hf] = make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]),
                                       __uint_as_float(x[2]), __uint_as_float(x[3]));
        }
    }
  };
  auto apply = [&](int pb, const Ops &o, floatx4 (&X)[CT][RT]) {
    floatx4 acc[CT][RT];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int t = 0; t < RT; ++t) acc[c][t] = o.st[c][t];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      bf16x8 ah[RT], al[RT];  // rows of M
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const float4 a0 = o.m[t][kb][0], a1 = o.m[t][kb][1];
        const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ah[t][e] = (__bf16)av[e];
          al[t][e] = (__bf16)(av[e] - (float)ah[t][e]);
        }
      }
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(&XH[pb][16 * c + j][32 * kb + 8 * g]);
        const bf16x8 bl = *reinterpret_cast<const bf16x8 *>(&XL[pb][16 * c + j][32 * kb + 8 * g]);
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          acc[c][t] = mfma_bf16_k32(al[t], bh, acc[c][t]);
          acc[c][t] = mfma_bf16_k32(ah[t], bl, acc[c][t]);
          acc[c][t] = mfma_bf16_k32(ah[t], bh, acc[c][t]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int t = 0; t < RT; ++t) X[c][t] = acc[c][t];
  };

  floatx4 X[CT][RT];
  int i0;  // first pair applied
  if (sc.mode == 1) {
    const float *P = pair_at(first);
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) X[c][t][r] = P[row_of(t, r) * (2 * D) + col_of(c)];
    i0 = first + 1;
  } else {
    const float *src = sc.init ? sc.init + ((int64_t)chain * sc.H + h) * (D * D) : nullptr;
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) X[c][t][r] = src ? src[row_of(t, r) * D + col_of(c)] : 0.f;
    i0 = first;
  }
  share(0, X);
  Ops ops[2];
  if (i0 < last) load_ops(i0, ops[0]);
  __syncthreads();

  // step n applies pair i0 + n, reading X from XT[n & 1] and sharing the result
  // in XT[(n + 1) & 1]; one barrier per step.  (The prefetch is unconditional --
  // the last step reloads its own operands -- so that the compiler's wait
  // counts never have to cover a path without it.)
  auto body = [&](int n, Ops &cur, Ops &nxt) {
    const int i = i0 + n;
    load_ops(min(i + 1, last - 1), nxt);
    if (sc.mode == 0) write_state(sc.states + ((int64_t)i * sc.H + h) * (D * D), D, X);
    apply(n & 1, cur, X);
    share((n + 1) & 1, X);
    lds_barrier();  // LDS only: the next step's operand loads stay in flight
  };
  const int nsteps = last - i0;
  int n = 0;
  for (; n + 1 < nsteps; n += 2) {
    body(n, ops[0], ops[1]);
    body(n + 1, ops[1], ops[0]);
  }
  if (n < nsteps) body(n, ops[0], ops[1]);
  if (sc.mode == 1) write_state(sc.composed + ((int64_t)chain * sc.H + h) * (D * 2 * D), 2 * D, X);
  if (final_write) write_state(sc.states + ((int64_t)max(first, last) * sc.H + h) * (D * D), D, X);
}

// A step is bound by the latency of its dependent loads and products, which
// more workgroups per compute unit hide: about four do best (the compose of
// 128 chains x 256 columns: 64-column slices, two per CU, 2.19 ms for the
// whole long-prefill step; 32-column slices, four per CU, 2.17 ms; 16-column
// slices, eight per CU, 2.26 ms).  So 64-column slices are taken only where
// they already give four per CU, 32-column slices where they give two, and
// chains too few for that (the scan of the segment or group pairs) take 16
// columns per workgroup in 8 waves of one row tile each: with one workgroup
// per compute unit, more waves with shorter MFMA chains and fewer loads each
// step faster (31 steps of the long prefill's pair scan: 74.6 us against
// 90.9 for 4 waves of two row tiles, identical results; loading the operands
// two steps ahead instead of one gained nothing).  (128-column slices of 8
// waves timed no faster.)
hipError_t launch_scan_chains(const ScanChains &sc, int n_cu, hipStream_t stream) {
  const int64_t units = (int64_t)sc.n_chains * sc.H;
  if (units * (sc.ncols / 64) >= 4 * (int64_t)n_cu) {
    hipLaunchKernelGGL((kda_scan_chains_kernel<4, 1>), dim3(scan_grid(units, sc.ncols / 64)), dim3(512),
                       0, stream, sc);
  } else if (units * (sc.ncols / 32) >= 2 * (int64_t)n_cu) {
    hipLaunchKernelGGL((kda_scan_chains_kernel<2, 2>), dim3(scan_grid(units, sc.ncols / 32)), dim3(256),
                       0, stream, sc);
  } else {
    hipLaunchKernelGGL((kda_scan_chains_kernel<1, 1>), dim3(scan_grid(units, sc.ncols / 16)), dim3(512),
                       0, stream, sc);
  }
  return hipGetLastError();
}

hipError_t launch_pair_scan(const float *pairs, const float *S0, const int32_t *cu, int N,
                            int H, int n_seg, int64_t seg_len, float *entry, hipStream_t stream) {
  hipLaunchKernelGGL(kda_pair_scan_kernel, dim3(scan_grid(H, 8)), dim3(SCAN_THREADS), 0, stream,
                     pairs, S0, cu, N, H, n_seg, seg_len, entry);
  return hipGetLastError();
}

}  // namespace kda
