// Runs the host side of every libkda entry point -- validation, segment and
// workspace planning, document order -- on the CPU, against the stubbed HIP
// runtime of hip_stubs.cpp.  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_sanitizers.py.  Device pointers are
// fake non-NULL values: the host code never dereferences them.  Prints "ok"
// and exits 0 when every status is the expected one.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "kda.h"

extern int g_launches;

static int failures = 0;
#define EXPECT(call, want)                                                                   \
  do {                                                                                       \
    const int got_ = (call);                                                                 \
    if (got_ != (want)) {                                                                    \
      std::printf("line %d: got %d, want %d (%s)\n", __LINE__, got_, (int)(want),            \
                  kda_last_error());                                                         \
      ++failures;                                                                            \
    }                                                                                        \
  } while (0)

int main() {
  alignas(256) char dev_mem[256];  // stands in for device pointers; never dereferenced
  void *F = dev_mem;
  float *Ff = reinterpret_cast<float *>(dev_mem);
  const int32_t *Fi = reinterpret_cast<const int32_t *>(dev_mem);
  const int H = 4;

  // ---- prefill: rejections (nothing launched) ----
  const int launches0 = g_launches;
  EXPECT(kda_chunk_fwd(nullptr, F, F, F, F, nullptr, -5.f, nullptr, nullptr, nullptr, 1, 256, H,
                       128, 128, KDA_BF16, 0, F, nullptr, nullptr, 0, nullptr),
         KDA_ERR_NULL);
  EXPECT(kda_chunk_fwd(F, F, F, F, F, nullptr, -6.f, nullptr, nullptr, nullptr, 1, 256, H, 128,
                       128, KDA_BF16, 0, F, nullptr, nullptr, 0, nullptr),
         KDA_ERR_GATE_BOUND);
  EXPECT(kda_chunk_fwd(F, F, F, F, F, nullptr, -5.f, nullptr, nullptr, nullptr, 1, 256, 65536, 128,
                       128, KDA_BF16, 0, F, nullptr, nullptr, 0, nullptr),
         KDA_ERR_SHAPE);
  {
    const int32_t bad[4] = {0, 100, 50, 256};  // not monotone
    EXPECT(kda_chunk_fwd(F, F, F, F, F, nullptr, -5.f, nullptr, Fi, bad, 3, 256, H, 128, 128,
                         KDA_BF16, 0, F, nullptr, nullptr, 0, nullptr),
           KDA_ERR_SEQLENS);
  }
  EXPECT(kda_chunk_fwd(F, F, F, F, F, nullptr, -5.f, nullptr, nullptr, nullptr, 1, 256, H, 128,
                       128, KDA_BF16, 0, F, nullptr, F, 16, nullptr),
         KDA_ERR_WORKSPACE);
  if (g_launches != launches0) {
    std::printf("a rejected call launched a kernel\n");
    ++failures;
  }

  // ---- prefill: valid calls reach the (failing) launch ----
  std::vector<int32_t> cu = {0};
  for (int d = 0; d < 300; ++d) cu.push_back(cu.back() + (d % 7 == 0 ? 0 : 37 * (d % 11) + 1));
  const int N = (int)cu.size() - 1;
  const int64_t T = cu.back();
  const size_t ws = kda_chunk_fwd_workspace_size(N, T, H, 128, 128);
  EXPECT(kda_chunk_fwd(F, F, F, F, F, Ff, -5.f, Ff, Fi, cu.data(), N, T, H, 128, 128, KDA_BF16, 0,
                       F, Ff, F, ws, nullptr),
         KDA_ERR_HIP);
  EXPECT(kda_chunk_fwd(F, F, F, F, F, Ff, -5.f, Ff, Fi, cu.data(), N, T, H, 128, 128,
                       KDA_BF16 | KDA_RAW_INPUTS, 0, F, Ff, F, ws, nullptr),
         KDA_ERR_HIP);
  EXPECT(kda_chunk_fwd(F, F, F, F, F, Ff, -5.f, Ff, Fi, cu.data(), N, T, H, 128, 128, KDA_F32,
                       KDA_COMPUTE_F32, F, Ff, nullptr, 0, nullptr),
         KDA_ERR_HIP);
  EXPECT(kda_chunk_fwd_unbounded(F, F, F, F, F, Ff, Ff, Fi, cu.data(), N, T, H, 128, 128, KDA_BF16,
                                 F, Ff, F, ws, nullptr),
         KDA_ERR_HIP);
  // the fused kernel: raw inputs, the unbounded gate, fp32 inputs
  EXPECT(kda_chunk_fwd(F, F, F, F, F, Ff, -5.f, Ff, Fi, cu.data(), N, T, H, 128, 128,
                       KDA_BF16 | KDA_RAW_INPUTS, 0, F, Ff, nullptr, 0, nullptr),
         KDA_ERR_HIP);
  EXPECT(kda_chunk_fwd(F, F, F, F, F, Ff, -5.f, Ff, Fi, cu.data(), N, T, H, 128, 128,
                       KDA_F32 | KDA_RAW_INPUTS, 0, F, Ff, nullptr, 0, nullptr),
         KDA_ERR_HIP);
  EXPECT(kda_chunk_fwd(F, F, F, F, F, Ff, -5.f, Ff, Fi, cu.data(), N, T, H, 128, 128,
                       KDA_BF16 | KDA_RAW_INPUTS, KDA_COMPUTE_F32, F, Ff, nullptr, 0, nullptr),
         KDA_ERR_UNSUPPORTED);  // bf16 inputs normalised into fp32 arithmetic
  EXPECT(kda_chunk_fwd_unbounded(F, F, F, F, F, Ff, Ff, Fi, cu.data(), N, T, H, 128, 128, KDA_BF16,
                                 F, Ff, nullptr, 0, nullptr),
         KDA_ERR_HIP);
  EXPECT(kda_chunk_fwd_unbounded(F, F, F, F, F, Ff, Ff, Fi, cu.data(), N, T, H, 128, 128,
                                 KDA_F32 | KDA_RAW_INPUTS, F, Ff, nullptr, 0, nullptr),
         KDA_ERR_HIP);
  {
    const int interval = 128;
    const size_t nck = kda_checkpoint_count(N, T, interval);
    EXPECT(kda_chunk_fwd_checkpoints(F, F, F, F, F, Ff, -5.f, Ff, Fi, cu.data(), N, T, H, 128, 128,
                                     KDA_BF16, interval, Ff, nck * H * 128 * 128 * 4, F, Ff, F, ws,
                                     nullptr),
           KDA_ERR_HIP);
  }
  EXPECT(kda_chunk_prep(F, F, F, F, Ff, -5.f, Fi, cu.data(), N, T, H, 128, 128, KDA_BF16, F, ws,
                        nullptr),
         KDA_ERR_HIP);
  // KDA_UNBOUNDED_GATE: g_min is neither used nor checked (-7 would be refused
  // by the bounded gate) on every prefill entry point and path; decode refuses it
  {
    const int32_t U = KDA_UNBOUNDED_GATE;
    EXPECT(kda_chunk_fwd(F, F, F, F, F, Ff, -7.f, Ff, Fi, cu.data(), N, T, H, 128, 128,
                         KDA_BF16, 0, F, Ff, F, ws, nullptr),
           KDA_ERR_GATE_BOUND);
    EXPECT(kda_chunk_fwd(F, F, F, F, F, Ff, -7.f, Ff, Fi, cu.data(), N, T, H, 128, 128,
                         KDA_BF16 | U, 0, F, Ff, F, ws, nullptr),
           KDA_ERR_HIP);  // two kernels
    EXPECT(kda_chunk_fwd(F, F, F, F, F, Ff, -7.f, Ff, Fi, cu.data(), N, T, H, 128, 128,
                         KDA_BF16 | U | KDA_RAW_INPUTS, 0, F, Ff, nullptr, 0, nullptr),
           KDA_ERR_HIP);  // fused
    EXPECT(kda_chunk_fwd(F, F, F, F, F, Ff, -7.f, Ff, Fi, cu.data(), N, T, H, 128, 128,
                         KDA_F32 | U, 0, F, Ff, nullptr, 0, nullptr),
           KDA_ERR_HIP);  // fp32
    EXPECT(kda_chunk_fwd_noalloc(F, F, F, F, F, Ff, -7.f, Ff, Fi, cu.data(), N, T, H, 128, 128,
                                 KDA_BF16 | U, F, Ff, nullptr),
           KDA_ERR_HIP);
    const size_t nck = kda_checkpoint_count(N, T, 128);
    EXPECT(kda_chunk_fwd_checkpoints(F, F, F, F, F, Ff, -7.f, Ff, Fi, cu.data(), N, T, H, 128, 128,
                                     KDA_BF16 | U, 128, Ff, nck * H * 128 * 128 * 4, F, Ff, F, ws,
                                     nullptr),
           KDA_ERR_HIP);
    EXPECT(kda_chunk_prep(F, F, F, F, Ff, -7.f, Fi, cu.data(), N, T, H, 128, 128, KDA_BF16 | U, F,
                          ws, nullptr),
           KDA_ERR_HIP);
    EXPECT(kda_chunk_recurrence(F, Ff, Fi, cu.data(), N, T, H, 128, 128, KDA_BF16 | U, F, ws, F,
                                Ff, nullptr),
           KDA_ERR_HIP);  // the flag changes nothing here
    for (int32_t dt : {KDA_BF16, KDA_F32}) {
      const size_t sws = kda_segment_scan_workspace_size(N, T, H, 7, 128, 128);
      EXPECT(kda_segment_scan(F, F, F, F, F, Ff, -7.f, nullptr, Fi, cu.data(), N, T, H, 128, 128,
                              dt | U, 0, 7, F, Ff, F, sws, nullptr),
             KDA_ERR_HIP);
    }
    EXPECT(kda_decode_step(Ff, 8, nullptr, F, F, F, F, F, Fi, 4, F, F, F, F, F, Ff, -7.f, F,
                           nullptr, 8, H, 128, 128, KDA_BF16 | U, nullptr),
           KDA_ERR_HIP);
  }
  EXPECT(kda_chunk_recurrence(F, Ff, Fi, cu.data(), N, T, H, 128, 128, KDA_BF16, F, ws, F, Ff,
                              nullptr),
         KDA_ERR_HIP);
  // segment scan: several segment counts on both arithmetic paths
  for (int n_seg : {1, 3, 64, 257, 100000}) {
    const size_t sws = kda_segment_scan_workspace_size(N, T, H, n_seg, 128, 128);
    EXPECT(kda_segment_scan(F, F, F, F, F, Ff, -5.f, Ff, Fi, cu.data(), N, T, H, 128, 128,
                            KDA_BF16, 0, n_seg, F, Ff + 1, F, sws, nullptr),
           KDA_ERR_UNSUPPORTED);  // final_state overlaps initial_state
    EXPECT(kda_segment_scan(F, F, F, F, F, Ff, -5.f, nullptr, Fi, cu.data(), N, T, H, 128, 128,
                            KDA_BF16, 0, n_seg, F, Ff, F, sws, nullptr),
           KDA_ERR_HIP);
    EXPECT(kda_segment_scan(F, F, F, F, F, Ff, -5.f, nullptr, Fi, cu.data(), N, T, H, 128, 128,
                            KDA_F32, 0, n_seg, F, Ff, F, sws, nullptr),
           KDA_ERR_HIP);
    // raw inputs on either path, except bf16 inputs with fp32 arithmetic
    EXPECT(kda_segment_scan(F, F, F, F, F, Ff, -5.f, nullptr, Fi, cu.data(), N, T, H, 128, 128,
                            KDA_BF16 | KDA_RAW_INPUTS, 0, n_seg, F, Ff, F, sws, nullptr),
           KDA_ERR_HIP);
    EXPECT(kda_segment_scan(F, F, F, F, F, Ff, -5.f, nullptr, Fi, cu.data(), N, T, H, 128, 128,
                            KDA_F32 | KDA_RAW_INPUTS, 0, n_seg, F, Ff, F, sws, nullptr),
           KDA_ERR_HIP);
    EXPECT(kda_segment_scan(F, F, F, F, F, Ff, -5.f, nullptr, Fi, cu.data(), N, T, H, 128, 128,
                            KDA_BF16 | KDA_RAW_INPUTS, KDA_COMPUTE_F32, n_seg, F, Ff, F, sws,
                            nullptr),
           KDA_ERR_UNSUPPORTED);
    EXPECT(kda_segment_scan(F, F, F, F, F, Ff, -5.f, nullptr, Fi, cu.data(), N, T, H, 128, 128,
                            KDA_BF16, 0, n_seg, F, Ff, F, 1024, nullptr),
           KDA_ERR_WORKSPACE);
  }

  // ---- the no-allocation prefill: too large for its scratch, then a fit ----
  EXPECT(kda_chunk_fwd_noalloc(F, F, F, F, F, Ff, -5.f, nullptr, nullptr, nullptr, 1, 8192, 96,
                               128, 128, KDA_BF16, F, Ff, nullptr),
         KDA_ERR_WORKSPACE);
  EXPECT(kda_chunk_fwd_noalloc(F, F, F, F, F, Ff, -5.f, nullptr, nullptr, nullptr, 1, 8192, 4,
                               128, 128, KDA_F32, F, Ff, nullptr),
         KDA_ERR_UNSUPPORTED);
  EXPECT(kda_chunk_fwd_noalloc(F, F, F, F, F, Ff, -5.f, Ff, Fi, cu.data(), N, T, H, 128, 128,
                               KDA_BF16, F, Ff, nullptr),
         KDA_ERR_HIP);
  EXPECT(kda_chunk_fwd_noalloc(F, F, F, F, F, Ff, -5.f, Ff, Fi, cu.data(), N, T, H, 128, 128,
                               KDA_BF16, F, Ff, (void *)0x1000),
         KDA_ERR_HIP);  // a stream of the current device
  EXPECT(kda_chunk_fwd_noalloc(F, F, F, F, F, Ff, -5.f, Ff, Fi, cu.data(), N, T, H, 128, 128,
                               KDA_BF16, F, Ff, (void *)0x2000),
         KDA_ERR_UNSUPPORTED);  // a stream of another device

  // ---- decode ----
  EXPECT(kda_decode_step(Ff, 7, nullptr, F, F, F, F, F, Fi, 4, F, F, F, F, F, Ff, -5.f, F,
                         nullptr, 8, H, 128, 128, KDA_BF16, nullptr),
         KDA_ERR_SHAPE);  // pool smaller than N without slots
  EXPECT(kda_decode_step(Ff, 2, Fi, F, F, F, F, F, Fi, 4, F, F, F, F, F, Ff, -5.f, F, nullptr, 8,
                         H, 128, 128, KDA_BF16, nullptr),
         KDA_ERR_HIP);
  EXPECT(kda_decode_step_window(Ff, 8, nullptr, F, F, F, F, F, Fi, 4, F, F, F, F, F, F, F, F, F, F,
                                3, Ff, -5.f, F, F, nullptr, 8, H, 128, 128, KDA_F32, nullptr),
         KDA_ERR_HIP);
  EXPECT(kda_decode_step_window(Ff, 8, nullptr, F, F, F, F, F, Fi, 4, F, F, F, F, F, nullptr, F, F,
                                F, F, 3, Ff, -5.f, F, F, nullptr, 8, H, 128, 128, KDA_F32, nullptr),
         KDA_ERR_NULL);

  if (failures == 0) std::printf("ok\n");
  return failures == 0 ? 0 : 1;
}
