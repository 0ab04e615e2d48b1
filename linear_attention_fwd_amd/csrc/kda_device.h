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
    uint2 w;
    w.x = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
    w.y = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
    *reinterpret_cast<uint2 *>(p) = w;
  }
};

// ---- buffer-resource access -------------------------------------------------
// Raw buffer loads/stores split an address into a per-lane VGPR offset and a
// wave-uniform SGPR offset.  The kernels keep 128 x 128 state tiles in MFMA
// accumulator layout; with plain pointers every element's 64-bit address is a
// separate loop-invariant value the compiler hoists and keeps live, with buffer
// access only one lane offset stays in a VGPR.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base) {
  // stride 0, full 31-bit range, gfx9 raw-buffer data format word
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, 0x7FFFFFFF, 0x00020000);
}
__device__ __forceinline__ float buf_ld_f32(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ void buf_st_f32(__amdgpu_buffer_rsrc_t r, float x, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, voff, soff, 0);
}

// A 128-row state slice in accumulator layout: tile[m][n][r] is row
// 16m + 4g + r, column col0 + 16n + j of a row-major matrix with `ld` columns.
template <int NT>
__device__ __forceinline__ void state_load(floatx4 (&S)[8][NT], const float *base, int ld,
                                           int col0, int g, int j) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(base);
  const int voff = (4 * g * ld + col0 + j) * 4;
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[m][n][e] = buf_ld_f32(r, voff, ((16 * m + e) * ld + 16 * n) * 4);
}
template <int NT>
__device__ __forceinline__ void state_store(const floatx4 (&S)[8][NT], float *base, int ld,
                                            int col0, int g, int j) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(base);
  const int voff = (4 * g * ld + col0 + j) * 4;
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int e = 0; e < 4; ++e) buf_st_f32(r, S[m][n][e], voff, ((16 * m + e) * ld + 16 * n) * 4);
}

// Bounded gate of equation (5) ("序列维度（下）", section "K3 的改动：下界衰减"):
// g = g_min * sigmoid(exp(A_h) * z).  `escale` = exp(A_h) is precomputed.
__device__ __forceinline__ float kda_gate(float z, float escale, float g_min) {
  const float x = escale * z;
  return g_min * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

}  // namespace kda
