// kda_prefill.hip -- fused chunkwise KDA prefill for gfx950 (no workspace): the
// kernel (kda_prefill_kernel.h) with the bounded gate on inputs as given, its
// launcher, and the final states of empty documents.
#include "kda_prefill_kernel.h"

namespace kda {

// final_state[d] = initial_state[d] (or 0) for empty documents
__global__ void kda_copy_empty_kernel(const int32_t *cu, int64_t T, const float *init, float *fin,
                                      int H) {
  const int d = blockIdx.x / H, h = blockIdx.x % H;
  const int64_t len = cu ? (int64_t)cu[d + 1] - cu[d] : T;
  if (len != 0) return;
  const int64_t base = ((int64_t)d * H + h) * (D * D);
  for (int x = threadIdx.x; x < D * D; x += blockDim.x) fin[base + x] = init ? init[base + x] : 0.f;
}

// The unbounded gate and raw inputs: kda_prefill_ext.hip.
hipError_t launch_fwd_ext(const FwdParams &p, bool bf16_in, bool f32_compute, bool unb, bool raw,
                          hipStream_t stream);

hipError_t launch_fwd(FwdParams p, bool bf16_in, bool f32_compute, int gate, bool raw,
                      hipStream_t stream) {
  // slices of 64 state columns per (item, head), 16 per wave: two for the
  // 128 value columns, four for the [S~ | M] pair columns
  p.nsplit = (p.mode == 2) ? 4 : 2;
  const bool unb = gate == GATE_SOFTPLUS;
  if (unb || raw) return launch_fwd_ext(p, bf16_in, f32_compute, unb, raw, stream);
  if (bf16_in)
    return f32_compute ? launch_fwd_t<bf16_t, true, false, false>(p, stream)
                       : launch_fwd_t<bf16_t, false, false, false>(p, stream);
  return f32_compute ? launch_fwd_t<float, true, false, false>(p, stream)
                     : launch_fwd_t<float, false, false, false>(p, stream);
}

hipError_t launch_copy_empty(const int32_t *cu, int64_t T, const float *init, float *fin, int N,
                             int H, hipStream_t stream) {
  hipLaunchKernelGGL(kda_copy_empty_kernel, dim3((unsigned)(N * H)), dim3(256), 0, stream, cu, T,
                     init, fin, H);
  return hipGetLastError();
}

}  // namespace kda
