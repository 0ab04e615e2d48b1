// kda_device.h -- device-side helpers shared by the KDA kernels (gfx950 only).
//
// MFMA lane layouts used throughout (64-lane wavefront, lane l, g = l / 16,
// j = l % 16):
//   v_mfma_f32_16x16x32_bf16 : A[i = j][k = 8g + e], B[k = 8g + e][n = j], e = 0..7
//   v_mfma_f32_16x16x16_bf16 : A[i = j][k = 4g + e], B[k = 4g + e][n = j], e = 0..3
//   v_mfma_f32_16x16x4_f32   : A[i = j][k = g],      B[k = g][n = j]
//   accumulator (all three)   : D[m = 4g + r][n = j], r = 0..3
// The hardware pairs A and B by (lane group g, element e); which logical k that
// slot carries is free as long as both operands agree.  The kernels use this to
// feed accumulator tiles straight back as B operands: the 16x16x32 slot (g, e)
// carries row 4g + e of the first 16-row tile for e < 4 and row 4g + e - 4 of
// the second tile for e >= 4 (see kperm32 below); A operands stored in LDS use
// the same permuted order along k.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
// fp32 -> bf16 (round to nearest even), two values per v_cvt_pk_bf16_f32
__device__ __forceinline__ bf16x4 to_bf16x4(floatx4 x) { return __builtin_convertvector(x, bf16x4); }
__device__ __forceinline__ bf16x8 to_bf16x8(floatx8 x) { return __builtin_convertvector(x, bf16x8); }
typedef uint16_t bf16_t;  // storage type of bf16 tensors in global memory

constexpr int D = 128;       // d_k = d_v
constexpr int CH = 64;       // chunk length C
constexpr int SUB = 16;      // subtile length

// Position of logical index x (0..31) of a 32-wide k block inside the MFMA
// k order (slot 8g + e).  Inverse of the mapping in the header comment.
__host__ __device__ constexpr int kperm32(int x) {
  return (x < 16) ? ((x >> 2) * 8 + (x & 3)) : (((x - 16) >> 2) * 8 + 4 + (x & 3));
}
// Permuted position inside a row whose k axis is a multiple of 32.
__host__ __device__ constexpr int kperm(int x) { return (x & ~31) + kperm32(x & 31); }

__device__ __forceinline__ floatx4 mfma_bf16_k32(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma_bf16_k16(bf16x4 a, bf16x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma_f32_k4(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
  return __uint_as_float(((uint32_t)x) << 16);
}
__device__ __forceinline__ bf16_t f32_to_bf16(float x) {
  __bf16 b = (__bf16)x;  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(bf16_t, b);
}

// ---- element loads/stores for the two input dtypes ------------------------
template <typename T> struct io;
template <> struct io<float> {
  // raw (not yet converted) register images, so loads can be issued early
  struct raw8 { float4 a, b; };
  typedef float raw1;
  static __device__ __forceinline__ raw8 ld8(const float *p) {
    return raw8{*reinterpret_cast<const float4 *>(p), *reinterpret_cast<const float4 *>(p + 4)};
  }
  static __device__ __forceinline__ void cvt8(const raw8 &r, float *x) {
    x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
    x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
  }
  static __device__ __forceinline__ raw1 ld1(const float *p) { return *p; }
  static __device__ __forceinline__ float cvt1(raw1 r) { return r; }
  // 8 consecutive elements
  static __device__ __forceinline__ void load8(const float *p, float *x) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  static __device__ __forceinline__ void load4(const float *p, float *x) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  }
  static __device__ __forceinline__ float load1(const float *p) { return *p; }
  static __device__ __forceinline__ void store1(float *p, float v) { *p = v; }
  static __device__ __forceinline__ void store4(float *p, const float *x) {
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
};
template <> struct io<bf16_t> {
  struct raw8 { uint4 a; };
  typedef bf16_t raw1;
  static __device__ __forceinline__ raw8 ld8(const bf16_t *p) {
    return raw8{*reinterpret_cast<const uint4 *>(p)};
  }
  static __device__ __forceinline__ void cvt8(const raw8 &r, float *x) {
    const uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ raw1 ld1(const bf16_t *p) { return *p; }
  static __device__ __forceinline__ float cvt1(raw1 r) { return bf16_to_f32(r); }
  static __device__ __forceinline__ void load8(const bf16_t *p, float *x) {
    const uint4 a = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void load4(const bf16_t *p, float *x) {
    const uint2 a = *reinterpret_cast<const uint2 *>(p);
    x[0] = __uint_as_float(a.x << 16);
    x[1] = __uint_as_float(a.x & 0xFFFF0000u);
    x[2] = __uint_as_float(a.y << 16);
    x[3] = __uint_as_float(a.y & 0xFFFF0000u);
  }
  static __device__ __forceinline__ float load1(const bf16_t *p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store1(bf16_t *p, float v) { *p = f32_to_bf16(v); }
  static __device__ __forceinline__ void store4(bf16_t *p, const float *x) {
    *reinterpret_cast<bf16x4 *>(p) = to_bf16x4(floatx4{x[0], x[1], x[2], x[3]});
  }
};

// ---- wave-uniform values ------------------------------------------------------
// Values the compiler cannot prove uniform (loaded through vector memory) are
// re-read from the first lane, so buffer descriptors built from them stay in
// SGPRs instead of being wrapped in per-lane loops.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uni64(int64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
template <typename T> __device__ __forceinline__ T *uniptr(T *p) {
  return reinterpret_cast<T *>((uintptr_t)uni64((int64_t)(uintptr_t)p));
}

// ---- buffer-resource access -------------------------------------------------
// Raw buffer loads/stores take a per-lane VGPR offset from a wave-uniform base.
// `bytes` bounds the descriptor: loads past it return 0 and stores past it are
// dropped, which masks ragged chunk tails without branches.  All offsets used
// here go into the VGPR operand (the range check covers it).
// The base and size must be wave-uniform; they are re-read from the first lane
// so the descriptor is built in SGPRs even when they reach here through a
// branch merge the compiler cannot prove uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
  // stride 0, gfx9 raw-buffer data format word
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(uniptr(base)), 0, uni(bytes), 0x00020000);
}
__device__ __forceinline__ float buf_ld_f32(__amdgpu_buffer_rsrc_t r, int voff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}
__device__ __forceinline__ void buf_st_f32(__amdgpu_buffer_rsrc_t r, float x, int voff) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, voff, 0, 0);
}

// Global -> LDS copies that bypass registers.  A buffer load with the lds bit
// writes 16 bytes per lane at M0 + 16 * lane (M0 = the wave-uniform LDS byte
// address of the 1 KB block).  It is issued through inline asm: the compiler
// otherwise makes every later LDS read wait for all such copies in flight,
// including reads of a different buffer, which would serialise the double
// buffering.  The caller waits (wait_vmem) and synchronises before reading
// the copied data.
//
// The compiler does not insert the wait states the hardware needs in front of
// an asm memory instruction: a vector memory read of an SGPR that a VALU
// instruction (v_readfirstlane, which builds the descriptor) wrote needs 5,
// and an LDS-DMA load after an SALU write of M0 needs 1.  Every asm load here
// therefore starts with s_nop 4 (5 wait states).
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 rsrc_words(const void *base, int bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)uniptr(base);
  return i32x4{(int)(uint32_t)b, (int)((uint32_t)(b >> 32) & 0xFFFFu), uni(bytes), 0x00020000};
}
// No memory clobber: the target LDS buffer is not accessed by the compiler's
// code until a later barrier (which has one), and volatile asm keeps its order
// relative to the other asm statements here.
__device__ __forceinline__ void copy16_to_lds(i32x4 rsrc, uint32_t lds_addr, int voff) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc),
               "{m0}"(lds_addr));
}
// LDS byte address of a __shared__ object
template <typename T> __device__ __forceinline__ uint32_t lds_addr(T *p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)(p);
}
// One dword per lane from global memory into LDS (lane l -> lds_addr + 4 l).  Used
// to pull lines into L2 ahead of a later copy: the data lands in a scratch LDS
// area nobody reads.  Offsets past the descriptor's size fetch nothing.
__device__ __forceinline__ void touch4_to_lds(i32x4 rsrc, uint32_t lds_addr, int voff) {
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc),
               "{m0}"(lds_addr)
               : "memory");
}
// s_waitcnt vmcnt(0): all vector memory operations of this wave have completed
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(N): all but the N most recently issued vector memory
// operations of this wave have completed.  That holds for operations of one
// kind, which complete in issue order; loads and stores share the counter but
// not that order, so every caller has only loads (or only stores) in flight.
template <int N> __device__ __forceinline__ void wait_vmem_except_last() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier that orders LDS only: unlike __syncthreads() it does not
// wait for this wave's outstanding global memory operations.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <typename T> struct bufio;
template <> struct bufio<float> {
  static constexpr int ES = 4;
  struct raw8 { u32x4 a, b; };
  typedef uint32_t raw1;
  static __device__ __forceinline__ raw8 ld8(__amdgpu_buffer_rsrc_t r, int voff) {
    return raw8{__builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0),
                __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, 0, 0)};
  }
  static __device__ __forceinline__ void cvt8(const raw8 &x, float *y) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { y[i] = __uint_as_float(x.a[i]); y[4 + i] = __uint_as_float(x.b[i]); }
  }
  static __device__ __forceinline__ raw1 ld1(__amdgpu_buffer_rsrc_t r, int voff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
  }
  static __device__ __forceinline__ float cvt1(raw1 x) { return __uint_as_float(x); }
  static __device__ __forceinline__ void st1(__amdgpu_buffer_rsrc_t r, float x, int voff) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, voff, 0, 0);
  }
};
template <> struct bufio<bf16_t> {
  static constexpr int ES = 2;
  struct raw8 { u32x4 a; };
  typedef unsigned short raw1;
  static __device__ __forceinline__ raw8 ld8(__amdgpu_buffer_rsrc_t r, int voff) {
    return raw8{__builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0)};
  }
  static __device__ __forceinline__ void cvt8(const raw8 &x, float *y) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[2 * i] = __uint_as_float(x.a[i] << 16);
      y[2 * i + 1] = __uint_as_float(x.a[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ raw1 ld1(__amdgpu_buffer_rsrc_t r, int voff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0);
  }
  static __device__ __forceinline__ float cvt1(raw1 x) { return bf16_to_f32(x); }
  static __device__ __forceinline__ void st1(__amdgpu_buffer_rsrc_t r, float x, int voff) {
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(x), r, voff, 0, 0);
  }
};

// A 128 x 16 state slice in accumulator layout: S[m][r] is row 16m + 4g + r,
// column col0 + j of a row-major fp32 matrix with `ld` columns at `base`
// (a wave-uniform pointer).
__device__ __forceinline__ void state_load(floatx4 (&S)[8], const float *base, int ld, int col0,
                                           int g, int j) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(base, D * ld * 4);
  const int voff = (4 * g * ld + col0 + j) * 4;
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e) S[m][e] = buf_ld_f32(r, voff + (16 * m + e) * ld * 4);
}
__device__ __forceinline__ void state_store(const floatx4 (&S)[8], float *base, int ld, int col0,
                                            int g, int j) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(base, D * ld * 4);
  const int voff = (4 * g * ld + col0 + j) * 4;
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e) buf_st_f32(r, S[m][e], voff + (16 * m + e) * ld * 4);
}

// ---- XOR-swizzled LDS tiles -------------------------------------------------
// Row-major tile with COLS elements of E per row.  The 16-byte chunk c of row r
// is stored at chunk c ^ sw(r), so that the 16 rows an MFMA operand read touches
// at one column fall into distinct banks.
template <typename E, int COLS> struct Tile {
  static constexpr int EPC = 16 / (int)sizeof(E);          // elements per 16-byte chunk
  static constexpr int NCH = COLS / EPC;                    // chunks per row
  static __device__ __forceinline__ int sw(int r) {
    return NCH >= 16 ? (r & 15) : ((r >> 1) & (NCH - 1));
  }
  // element offset of logical (r, col); an access of up to one chunk starting at
  // col must not cross a chunk boundary
  static __device__ __forceinline__ int idx(int r, int col) {
    return r * COLS + (((col / EPC) ^ sw(r)) * EPC) + (col % EPC);
  }
};

// Bounded gate of equation (5) ("序列维度（下）", section "K3 的改动：下界衰减"),
// g = g_min * sigmoid(exp(A_h) z), returned in base-2 units (g * log2 e) so the
// decay factors are plain exp2.  c1 = -exp(A_h) * log2 e and gm = g_min * log2 e
// are precomputed; gm = 0 turns a padding row into "no decay".
__device__ __forceinline__ float kda_gate2(float z, float c1, float gm) {
  return gm * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(c1 * z));
}
// Unbounded gate that the same section gives for Kimi Linear (as in GDN and
// Mamba-2), g = -exp(A_h) softplus(z), in base-2 units: c1 = -exp(A_h) log2 e,
// or 0 for a padding row.  softplus(z) = max(z, 0) + ln(1 + e^-|z|), which
// cannot overflow.
__device__ __forceinline__ float kda_gate2_softplus(float z, float c1) {
  const float t = __builtin_amdgcn_exp2f(-1.4426950408889634f * fabsf(z));  // e^-|z|
  const float sp = fmaxf(z, 0.0f) + 0.6931471805599453f * __builtin_amdgcn_logf(1.0f + t);
  return c1 * sp;
}
// The same gate in natural-log units (decode path).
__device__ __forceinline__ float kda_gate(float z, float escale, float g_min) {
  const float x = escale * z;
  return g_min * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

}  // namespace kda
