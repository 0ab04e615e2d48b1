// kda_api.cpp -- C ABI of libkda.so: argument validation and kernel launches.
//
// Every check that the host can make happens before the first HIP call, so a
// rejected call enqueues nothing.  No exception crosses the ABI.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/kda.h"
#include "kda_launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kD = 128;
constexpr int kC = 64;  // chunk length
// The kernels address the rows of one 64-token chunk of one head with 32-bit
// byte offsets: up to 64 tokens x H heads x 128 channels x 4 bytes.
constexpr int kMaxHeads = 65535;
static_assert((int64_t)kC * kMaxHeads * kD * 4 <= (int64_t)INT32_MAX, "chunk offsets fit int32");
// One dispatch covers at most 2^32 - 1 work-items (grid x workgroup size).
// Every grid here is a fixed multiple of a unit count, which bounds the units;
// the bounds are checked before anything is enqueued:
//   prep: a 256-thread workgroup per (chunk slot, head);
//   recurrence and fused prefill: 512 work-items per (document, head) unit,
//     unit counts rounded up to a multiple of 8 (the recurrence takes one
//     workgroup per unit once the units fill the device);
//   segment pairs: 1024 per (segment, head); composing them: 2048 per
//     (segment group, head);
//   decode and the empty-document copy: a 256-thread workgroup per (sequence, head).
constexpr int64_t kMaxItems = 0xFFFFFFFFll;
constexpr int64_t kMaxSlotHeads = kMaxItems / 256;
constexpr int64_t kMaxDocHeads = kMaxItems / 512 / 8 * 8;
constexpr int64_t kMaxSegHeads = kMaxItems / 1024 / 8 * 8;
constexpr int64_t kMaxGroupHeads = kMaxItems / 2048 / 8 * 8;
constexpr int64_t kMaxSeqHeads = kMaxItems / 256;

// The KDA_RAW_INPUTS flag of a dtype argument; the element type is the rest.
bool take_raw_flag(int32_t &dtype) {
  const bool raw = (dtype & KDA_RAW_INPUTS) != 0;
  dtype &= ~KDA_RAW_INPUTS;
  return raw;
}
// The KDA_UNBOUNDED_GATE flag of a dtype argument, as the gate map it selects.
int take_gate_flag(int32_t &dtype) {
  const bool unb = (dtype & KDA_UNBOUNDED_GATE) != 0;
  dtype &= ~KDA_UNBOUNDED_GATE;
  return unb ? kda::GATE_SOFTPLUS : kda::GATE_BOUNDED;
}
int raw_unsupported(const char *who) {
  return fail(KDA_ERR_UNSUPPORTED,
              "%s: raw inputs with fp32 arithmetic need fp32 inputs (bf16 inputs would be "
              "normalised into bf16 operands)", who);
}

// Sizes, dtype and document offsets shared by the prefill entry points.
int check_layout(const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, int32_t N, int64_t T,
                 int32_t H, int32_t dk, int32_t dv, int32_t dtype) {
  if (dk != kD || dv != kD) return fail(KDA_ERR_SHAPE, "only d_k = d_v = 128 is supported (got %d, %d)", dk, dv);
  if (H <= 0) return fail(KDA_ERR_SHAPE, "H must be positive (got %d)", H);
  if (H > kMaxHeads) return fail(KDA_ERR_SHAPE, "H must be at most %d (got %d)", kMaxHeads, H);
  if (T < 0) return fail(KDA_ERR_SHAPE, "T must be >= 0");
  if (N <= 0) return fail(KDA_ERR_SHAPE, "N must be >= 1 (got %d)", N);
  if (T > (int64_t)INT32_MAX) return fail(KDA_ERR_SHAPE, "T must fit int32 offsets");
  if ((int64_t)N * H > kMaxDocHeads)
    return fail(KDA_ERR_SHAPE, "N * H = %lld exceeds %lld (one launch)", (long long)N * H,
                (long long)kMaxDocHeads);
  if (kda::n_chunk_slots(T, N) * H > kMaxSlotHeads)
    return fail(KDA_ERR_SHAPE, "chunk slots * H = %lld exceeds %lld (one launch)",
                (long long)(kda::n_chunk_slots(T, N) * H), (long long)kMaxSlotHeads);
  if (dtype != KDA_F32 && dtype != KDA_BF16) return fail(KDA_ERR_DTYPE, "unknown dtype %d", dtype);
  if (cu_seqlens) {
    if (!cu_seqlens_host)
      return fail(KDA_ERR_SEQLENS, "cu_seqlens_host is required with cu_seqlens");
    if (cu_seqlens_host[0] != 0) return fail(KDA_ERR_SEQLENS, "cu_seqlens[0] must be 0");
    for (int32_t n = 0; n < N; ++n)
      if (cu_seqlens_host[n + 1] < cu_seqlens_host[n])
        return fail(KDA_ERR_SEQLENS, "cu_seqlens must be non-decreasing (at %d)", n);
    if ((int64_t)cu_seqlens_host[N] != T)
      return fail(KDA_ERR_SEQLENS, "cu_seqlens[N] = %d but T = %lld", cu_seqlens_host[N], (long long)T);
  } else if (N != 1) {
    return fail(KDA_ERR_SEQLENS, "cu_seqlens is required when N > 1");
  }
  return KDA_OK;
}

int check_gate(float g_min) {
  if (!(g_min >= -5.0f && g_min < 0.0f))
    return fail(KDA_ERR_GATE_BOUND, "g_min must lie in [-5, 0) (got %g)", (double)g_min);
  return KDA_OK;
}

// Shared validation of the full prefill entry points.
int check_prefill(const void *q, const void *k, const void *v, const void *g_logits,
                  const void *beta, float g_min, const int32_t *cu_seqlens,
                  const int32_t *cu_seqlens_host, int32_t N, int64_t T, int32_t H, int32_t dk,
                  int32_t dv, int32_t dtype, int32_t compute, const void *o, int gate) {
  if (T > 0 && (!q || !k || !v || !g_logits || !beta || !o))
    return fail(KDA_ERR_NULL, "q, k, v, g_logits, beta and o must be non-NULL when T > 0");
  int rc = check_layout(cu_seqlens, cu_seqlens_host, N, T, H, dk, dv, dtype);
  if (rc != KDA_OK) return rc;
  if (compute != KDA_COMPUTE_AUTO && compute != KDA_COMPUTE_F32)
    return fail(KDA_ERR_DTYPE, "unknown compute mode %d", compute);
  return gate == kda::GATE_SOFTPLUS ? KDA_OK : check_gate(g_min);  // the unbounded gate has no g_min
}

// Workspace of the two-kernel path (chunk images).
int check_image_workspace(const void *workspace, size_t workspace_bytes, int64_t T, int32_t N,
                          int32_t H) {
  if (T == 0) return KDA_OK;
  const size_t need = kda::split_workspace_bytes(T, N, H);
  if (!workspace || workspace_bytes < need)
    return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
  if (((uintptr_t)workspace & 255u) != 0) return fail(KDA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return KDA_OK;
}

// The recurrence takes the documents longest first (an order the prep kernel
// launcher writes into the workspace) unless their chunk counts already do
// not increase, when the order would be the input order.
bool needs_doc_order(const int32_t *cu_host, int32_t N) {
  if (!cu_host || N < 2) return false;
  int64_t prev = INT64_MAX;
  for (int32_t d = 0; d < N; ++d) {
    const int64_t c = ((int64_t)cu_host[d + 1] - cu_host[d] + kC - 1) / kC;
    if (c > prev) return true;
    prev = c;
  }
  return false;
}

kda::SplitParams split_params(const void *q, const void *k, const void *v, const void *g_logits,
                              const void *beta, const float *A_log, float g_min,
                              const float *initial_state, const int32_t *cu_seqlens,
                              const int32_t *cu_host, int32_t N, int64_t T, int32_t H, void *o,
                              float *final_state, const void *ws) {
  kda::SplitParams p{};
  p.q = q; p.k = k; p.v = v; p.z = g_logits; p.beta = beta;
  p.A_log = A_log; p.g_min = g_min;
  p.cu = cu_seqlens; p.N = N; p.T = T; p.H = H;
  p.init = initial_state; p.o = o; p.final_state = final_state;
  p.ws = const_cast<void *>(ws); p.n_slots = kda::n_chunk_slots(T, N);
  if (needs_doc_order(cu_host, N))
    p.order = (int32_t *)((char *)p.ws + kda::split_order_offset(T, N, H));
  return p;
}

bool has_empty_doc(const int32_t *cu_host, int32_t N, int64_t T) {
  if (!cu_host) return T == 0;
  for (int32_t n = 0; n < N; ++n)
    if (cu_host[n + 1] == cu_host[n]) return true;
  return false;
}

size_t scan_workspace(int64_t n_seg, int64_t H) {
  return (size_t)n_seg * H * kD * (3 * kD) * sizeof(float);  // pairs [., 2D] + entry [., D]
}

// Segment plans.  The fused path (fp32 arithmetic) cuts the tokens into n_seg
// equal ranges; the two-kernel path cuts the chunk slots into n_seg equal
// ranges.  Both clamp the count so that no segment is empty.
struct SegPlan {
  int64_t n_seg, len;  // number of segments and tokens (fused) or slots (two-kernel) per segment
};
SegPlan plan_segments(int64_t units, int64_t requested) {
  int64_t n = requested;
  if (n > units) n = units;
  if (n < 1) n = 1;
  const int64_t len = (units + n - 1) / n;
  return SegPlan{(units + len - 1) / len, len};
}
// The two-kernel path scans its segment pairs in two levels: groups of about
// sqrt(n_seg) consecutive pairs are composed into one pair each (in parallel)
// and the group pairs are scanned into the entry state of each group; the
// re-run then walks each group's segments back to back from that state.  The
// dependent chain is about 2 sqrt(n_seg) pair applications instead of n_seg.
int64_t scan_group_len(int64_t n_seg) {
  int64_t g = 1;
  while (g * g < n_seg) ++g;
  return g;
}
int64_t scan_groups(int64_t n_seg) {
  const int64_t g = scan_group_len(n_seg);
  return (n_seg + g - 1) / g;
}
// Chunk slots up to and including the last one that holds a chunk: the
// segments of the two-kernel path divide these (the slot after a document whose
// length is a multiple of 64, and the slots of trailing empty documents, hold
// none; leaving them out keeps the segments, and so the passes over them, as
// short as the requested count allows).
int64_t used_chunk_slots(int64_t T, int32_t N, const int32_t *cu_host) {
  for (int32_t d = N - 1; d >= 0; --d) {
    const int64_t a = cu_host ? cu_host[d] : 0, b = cu_host ? cu_host[d + 1] : T;
    if (b > a) return kda::first_slot(a, d) + (b - a + 63) / 64;
  }
  return 0;
}
// Most segments any plan over at most n_chunk_slots units can give:
// min(requested, units); and the most groups any of those segment counts gives
// (taken over all of them, so that the buffers fit whatever the group length).
int64_t max_split_segments(int64_t T, int32_t N, int64_t requested) {
  int64_t n_max = requested < 1 ? 1 : requested;
  if (n_max > kda::n_chunk_slots(T, N)) n_max = kda::n_chunk_slots(T, N);
  return n_max;
}
int64_t max_scan_groups(int64_t n_max) {
  int64_t m = 1;
  for (int64_t n = 1; n <= n_max; ++n)
    if (scan_groups(n) > m) m = scan_groups(n);
  return m;
}
// The two-kernel path's segment count for a request (n_segments <= 0: the
// default) and whether its pairs are scanned in one level.  By default each
// (segment, head) unit gets a compute unit: n = ceil(CUs / H) segments, one
// level (every segment its own group), while that keeps the scan's chain at
// 32 pairs or fewer; the group pairs are then the segment pairs, no pairs are
// composed, and the re-run's units fill the device.  (On the long prefill,
// T = 262144 with H = 8: 32 segments in one level, 2.02 ms, against 256 in two
// levels, 2.14 ms: the composition of 240 pairs costs more than a longer scan
// saves.)  Beyond 32, and for any count the caller gives, one segment per
// requested unit and two levels.
struct SplitRequest {
  int64_t n;
  bool one_level;
};
SplitRequest split_request(int32_t n_segments, int32_t H, int cus) {
  if (n_segments > 0) return SplitRequest{n_segments, false};
  const int64_t per_head = ((int64_t)cus + H - 1) / H;
  if (per_head <= 32) return SplitRequest{per_head, true};
  return SplitRequest{cus, false};
}
size_t split_scan_workspace(int64_t T, int32_t N, int32_t H, const SplitRequest &r) {
  const int64_t n_max = max_split_segments(T, N, r.n);
  const int64_t g_max = r.one_level ? n_max : max_scan_groups(n_max);
  // chunk images, segment pairs [., D, 2D], group pairs and group entry states
  return kda::split_workspace_bytes(T, N, H) + (size_t)n_max * H * kD * 2 * kD * sizeof(float) +
         scan_workspace(g_max, H);
}

}  // namespace

extern "C" {

const char *kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_NULL: return "KDA_ERR_NULL";
    case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE";
    case KDA_ERR_DTYPE: return "KDA_ERR_DTYPE";
    case KDA_ERR_GATE_BOUND: return "KDA_ERR_GATE_BOUND";
    case KDA_ERR_SEQLENS: return "KDA_ERR_SEQLENS";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    default: return "KDA_ERR_UNKNOWN";
  }
}

const char *kda_last_error(void) { return g_err; }

int kda_chunk_fwd(const void *q, const void *k, const void *v, const void *g_logits,
                  const void *beta, const float *A_log, float g_min,
                  const float *initial_state, const int32_t *cu_seqlens,
                  const int32_t *cu_seqlens_host, int32_t N, int64_t T, int32_t H,
                  int32_t dk, int32_t dv, int32_t dtype, int32_t compute, void *o,
                  float *final_state, void *workspace, size_t workspace_bytes, void *stream) {
  const bool raw = take_raw_flag(dtype);
  const int gate = take_gate_flag(dtype);
  int rc = check_prefill(q, k, v, g_logits, beta, g_min, cu_seqlens, cu_seqlens_host, N, T, H,
                         dk, dv, dtype, compute, o, gate);
  if (rc != KDA_OK) return rc;
  const bool f32c = compute == KDA_COMPUTE_F32 || dtype == KDA_F32;
  const bool split = workspace != nullptr && !f32c;
  if (raw && f32c && dtype == KDA_BF16) return raw_unsupported("kda_chunk_fwd");
  if (split) {
    rc = check_image_workspace(workspace, workspace_bytes, T, N, H);
    if (rc != KDA_OK) return rc;
  }
  hipStream_t st = (hipStream_t)stream;
  if (T > 0 && split) {
    kda::SplitParams p = split_params(q, k, v, g_logits, beta, A_log, g_min, initial_state,
                                      cu_seqlens, cu_seqlens_host, N, T, H, o, final_state,
                                      workspace);
    p.raw = raw;
    p.gate = gate;
    hipError_t e = kda::launch_chunk_prep(p, st);
    if (e == hipSuccess) e = kda::launch_chunk_recurrence(p, st);
    if (e != hipSuccess) return hip_fail(e, "kda_chunk_fwd launch");
  } else if (T > 0) {
    kda::FwdParams p{};
    p.q = q; p.k = k; p.v = v; p.z = g_logits; p.beta = beta;
    p.A_log = A_log; p.g_min = g_min;
    p.cu = cu_seqlens; p.N = N; p.T = T; p.H = H;
    p.mode = 0; p.n_items = N; p.seg_len = 0;
    p.item_init = initial_state; p.doc_init = nullptr;
    p.o = o; p.final_state = final_state;
    hipError_t e = kda::launch_fwd(p, dtype == KDA_BF16, f32c, gate, raw, st);
    if (e != hipSuccess) return hip_fail(e, "kda_chunk_fwd launch");
  }
  if (final_state && has_empty_doc(cu_seqlens_host, N, T)) {
    hipError_t e = kda::launch_copy_empty(cu_seqlens, T, initial_state, final_state, N, H, st);
    if (e != hipSuccess) return hip_fail(e, "kda_chunk_fwd empty documents");
  }
  return KDA_OK;
}

int kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const void *g_logits,
                          const void *beta, const float *A_log, float g_min,
                          const float *initial_state, const int32_t *cu_seqlens,
                          const int32_t *cu_seqlens_host, int32_t N, int64_t T, int32_t H,
                          int32_t dk, int32_t dv, int32_t dtype, void *o, float *final_state,
                          void *stream) {
  static_assert(KDA_NOALLOC_SCRATCH_BYTES == kda::NOALLOC_SCRATCH_BYTES, "documented limit");
  const bool raw = take_raw_flag(dtype);
  const int gate = take_gate_flag(dtype);
  int rc = check_prefill(q, k, v, g_logits, beta, g_min, cu_seqlens, cu_seqlens_host, N, T, H,
                         dk, dv, dtype, KDA_COMPUTE_AUTO, o, gate);
  if (rc != KDA_OK) return rc;
  if (dtype != KDA_BF16)
    return fail(KDA_ERR_UNSUPPORTED, "kda_chunk_fwd_noalloc runs the bf16 two-kernel path only");
  const size_t need = kda::split_workspace_bytes(T, N, H);
  if (need > kda::NOALLOC_SCRATCH_BYTES)
    return fail(KDA_ERR_WORKSPACE,
                "kda_chunk_fwd_noalloc: %zu bytes of scratch needed (N = %d, T = %lld, H = %d), "
                "%zu available; call kda_chunk_fwd with a workspace instead",
                need, N, (long long)T, H, kda::NOALLOC_SCRATCH_BYTES);
  hipStream_t st = (hipStream_t)stream;
  if (T > 0) {
    // The scratch is looked up on the current device and the kernels run on
    // the stream's: a stream of another device would get a foreign address.
    if (st) {
      int dev = 0;
      hipDevice_t sdev = 0;
      hipError_t e = hipGetDevice(&dev);
      if (e == hipSuccess) e = hipStreamGetDevice(st, &sdev);
      if (e != hipSuccess) return hip_fail(e, "kda_chunk_fwd_noalloc stream device");
      if (sdev != dev)
        return fail(KDA_ERR_UNSUPPORTED,
                    "kda_chunk_fwd_noalloc: the stream belongs to device %d, not to the current "
                    "device %d", (int)sdev, dev);
    }
    void *ws = nullptr;
    hipError_t e = kda::noalloc_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e, "kda_chunk_fwd_noalloc scratch address");
    kda::SplitParams p = split_params(q, k, v, g_logits, beta, A_log, g_min, initial_state,
                                      cu_seqlens, cu_seqlens_host, N, T, H, o, final_state, ws);
    p.raw = raw;
    p.gate = gate;
    e = kda::launch_chunk_prep(p, st);
    if (e == hipSuccess) e = kda::launch_chunk_recurrence(p, st);
    if (e != hipSuccess) return hip_fail(e, "kda_chunk_fwd_noalloc launch");
  }
  if (final_state && has_empty_doc(cu_seqlens_host, N, T)) {
    hipError_t e = kda::launch_copy_empty(cu_seqlens, T, initial_state, final_state, N, H, st);
    if (e != hipSuccess) return hip_fail(e, "kda_chunk_fwd_noalloc empty documents");
  }
  return KDA_OK;
}

size_t kda_checkpoint_count(int32_t N, int64_t T, int32_t interval) {
  if (N <= 0 || T < 0 || interval <= 0 || interval % kC != 0) return 0;
  return (size_t)((kda::n_chunk_slots(T, N) - 1) / (interval / kC) + 1);
}

int kda_chunk_fwd_checkpoints(const void *q, const void *k, const void *v, const void *g_logits,
                              const void *beta, const float *A_log, float g_min,
                              const float *initial_state, const int32_t *cu_seqlens,
                              const int32_t *cu_seqlens_host, int32_t N, int64_t T, int32_t H,
                              int32_t dk, int32_t dv, int32_t dtype, int32_t interval,
                              float *checkpoints, size_t checkpoint_bytes, void *o,
                              float *final_state, void *workspace, size_t workspace_bytes,
                              void *stream) {
  const bool raw = take_raw_flag(dtype);
  const int gate = take_gate_flag(dtype);
  int rc = check_prefill(q, k, v, g_logits, beta, g_min, cu_seqlens, cu_seqlens_host, N, T, H,
                         dk, dv, dtype, KDA_COMPUTE_AUTO, o, gate);
  if (rc != KDA_OK) return rc;
  if (dtype != KDA_BF16) return fail(KDA_ERR_UNSUPPORTED, "checkpoints are written by the bf16 two-kernel path only");
  if (interval <= 0 || interval % kC != 0)
    return fail(KDA_ERR_SHAPE, "checkpoint interval must be a positive multiple of %d tokens (got %d)", kC, interval);
  if (!checkpoints) return fail(KDA_ERR_NULL, "checkpoints must be non-NULL");
  const size_t need_ckpt = kda_checkpoint_count(N, T, interval) * (size_t)H * kD * kD * sizeof(float);
  if (checkpoint_bytes < need_ckpt)
    return fail(KDA_ERR_WORKSPACE, "checkpoint buffer of %zu bytes required (got %zu)", need_ckpt, checkpoint_bytes);
  rc = check_image_workspace(workspace, workspace_bytes, T, N, H);
  if (rc != KDA_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  if (T > 0) {
    kda::SplitParams p = split_params(q, k, v, g_logits, beta, A_log, g_min, initial_state,
                                      cu_seqlens, cu_seqlens_host, N, T, H, o, final_state,
                                      workspace);
    p.ckpt = checkpoints;
    p.ckpt_chunks = interval / kC;
    p.raw = raw;
    p.gate = gate;
    hipError_t e = kda::launch_chunk_prep(p, st);
    if (e == hipSuccess) e = kda::launch_chunk_recurrence(p, st);
    if (e != hipSuccess) return hip_fail(e, "kda_chunk_fwd_checkpoints launch");
  }
  if (final_state && has_empty_doc(cu_seqlens_host, N, T)) {
    hipError_t e = kda::launch_copy_empty(cu_seqlens, T, initial_state, final_state, N, H, st);
    if (e != hipSuccess) return hip_fail(e, "kda_chunk_fwd_checkpoints empty documents");
  }
  return KDA_OK;
}

int kda_chunk_fwd_unbounded(const void *q, const void *k, const void *v, const void *g_logits,
                            const void *beta, const float *A_log, const float *initial_state,
                            const int32_t *cu_seqlens, const int32_t *cu_seqlens_host, int32_t N,
                            int64_t T, int32_t H, int32_t dk, int32_t dv, int32_t dtype, void *o,
                            float *final_state, void *workspace, size_t workspace_bytes,
                            void *stream) {
  // kda_chunk_fwd with the unbounded gate and the arithmetic of the inputs:
  // bf16 inputs with a workspace take the two kernels, without one the fused
  // kernel; fp32 inputs take the fused kernel in fp32 arithmetic
  return kda_chunk_fwd(q, k, v, g_logits, beta, A_log, -5.0f, initial_state, cu_seqlens,
                       cu_seqlens_host, N, T, H, dk, dv, dtype | KDA_UNBOUNDED_GATE,
                       KDA_COMPUTE_AUTO, o, final_state, workspace, workspace_bytes, stream);
}

size_t kda_chunk_fwd_workspace_size(int32_t N, int64_t T, int32_t H, int32_t dk, int32_t dv) {
  if (N <= 0 || T < 0 || H <= 0 || dk != kD || dv != kD) return 0;
  return kda::split_workspace_bytes(T, N, H);
}

int kda_chunk_prep(const void *q, const void *k, const void *g_logits, const void *beta,
                   const float *A_log, float g_min, const int32_t *cu_seqlens,
                   const int32_t *cu_seqlens_host, int32_t N, int64_t T, int32_t H, int32_t dk,
                   int32_t dv, int32_t dtype, void *workspace, size_t workspace_bytes,
                   void *stream) {
  const bool raw = take_raw_flag(dtype);
  const int gate = take_gate_flag(dtype);
  if (T > 0 && (!q || !k || !g_logits || !beta))
    return fail(KDA_ERR_NULL, "q, k, g_logits and beta must be non-NULL when T > 0");
  int rc = check_layout(cu_seqlens, cu_seqlens_host, N, T, H, dk, dv, dtype);
  if (rc == KDA_OK && gate == kda::GATE_BOUNDED) rc = check_gate(g_min);
  if (rc != KDA_OK) return rc;
  if (dtype != KDA_BF16) return fail(KDA_ERR_UNSUPPORTED, "kda_chunk_prep takes bf16 inputs only");
  rc = check_image_workspace(workspace, workspace_bytes, T, N, H);
  if (rc != KDA_OK || T == 0) return rc;
  kda::SplitParams p = split_params(q, k, nullptr, g_logits, beta, A_log, g_min, nullptr,
                                    cu_seqlens, cu_seqlens_host, N, T, H, nullptr, nullptr,
                                    workspace);
  p.raw = raw;
  p.gate = gate;
  hipError_t e = kda::launch_chunk_prep(p, (hipStream_t)stream);
  return e == hipSuccess ? KDA_OK : hip_fail(e, "kda_chunk_prep launch");
}

int kda_chunk_recurrence(const void *v, const float *initial_state, const int32_t *cu_seqlens,
                         const int32_t *cu_seqlens_host, int32_t N, int64_t T, int32_t H,
                         int32_t dk, int32_t dv, int32_t dtype, const void *workspace,
                         size_t workspace_bytes, void *o, float *final_state, void *stream) {
  if (T > 0 && (!v || !o)) return fail(KDA_ERR_NULL, "v and o must be non-NULL when T > 0");
  take_raw_flag(dtype);   // the recurrence reads v and the chunk images only:
  take_gate_flag(dtype);  // neither flag changes anything here
  int rc = check_layout(cu_seqlens, cu_seqlens_host, N, T, H, dk, dv, dtype);
  if (rc != KDA_OK) return rc;
  if (dtype != KDA_BF16) return fail(KDA_ERR_UNSUPPORTED, "kda_chunk_recurrence takes bf16 inputs only");
  rc = check_image_workspace(workspace, workspace_bytes, T, N, H);
  if (rc != KDA_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  if (T > 0) {
    const kda::SplitParams p = split_params(nullptr, nullptr, v, nullptr, nullptr, nullptr, -5.0f,
                                            initial_state, cu_seqlens, cu_seqlens_host, N, T, H,
                                            o, final_state, workspace);
    hipError_t e = kda::launch_chunk_recurrence(p, st);
    if (e != hipSuccess) return hip_fail(e, "kda_chunk_recurrence launch");
  }
  if (final_state && has_empty_doc(cu_seqlens_host, N, T)) {
    hipError_t e = kda::launch_copy_empty(cu_seqlens, T, initial_state, final_state, N, H, st);
    if (e != hipSuccess) return hip_fail(e, "kda_chunk_recurrence empty documents");
  }
  return KDA_OK;
}

int kda_default_segments(void) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(KDA_ERR_HIP, "hipGetDevice failed");
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return fail(KDA_ERR_HIP, "cannot query the compute-unit count");
  return cus;
}

size_t kda_segment_scan_workspace_size(int32_t N, int64_t T, int32_t H, int32_t n_segments,
                                       int32_t dk, int32_t dv) {
  if (N <= 0 || T < 0 || H <= 0 || dk != kD || dv != kD) return 0;
  int cus = 0;
  if (n_segments <= 0) {
    cus = kda_default_segments();
    if (cus < 0) return 0;
  }
  // enough for either arithmetic path
  const int64_t req = n_segments > 0 ? n_segments : cus;
  const size_t fused = scan_workspace(plan_segments(T > 0 ? T : 1, req).n_seg, H);
  const size_t split = split_scan_workspace(T, N, H, split_request(n_segments, H, cus));
  return fused > split ? fused : split;
}

int kda_segment_scan(const void *q, const void *k, const void *v, const void *g_logits,
                     const void *beta, const float *A_log, float g_min,
                     const float *initial_state, const int32_t *cu_seqlens,
                     const int32_t *cu_seqlens_host, int32_t N, int64_t T, int32_t H,
                     int32_t dk, int32_t dv, int32_t dtype, int32_t compute,
                     int32_t n_segments, void *o, float *final_state, void *workspace,
                     size_t workspace_bytes, void *stream) {
  const bool raw = take_raw_flag(dtype);
  const int gate = take_gate_flag(dtype);
  int rc = check_prefill(q, k, v, g_logits, beta, g_min, cu_seqlens, cu_seqlens_host, N, T, H,
                         dk, dv, dtype, compute, o, gate);
  if (rc != KDA_OK) return rc;
  if (final_state && initial_state) {
    // [N, H, D, D] fp32 each; any overlap is refused
    const uintptr_t bytes = (uintptr_t)N * H * kD * kD * sizeof(float);
    const uintptr_t f = (uintptr_t)final_state, i = (uintptr_t)initial_state;
    if (f < i + bytes && i < f + bytes)
      return fail(KDA_ERR_UNSUPPORTED, "kda_segment_scan: final_state must not overlap initial_state");
  }
  const bool f32c = compute == KDA_COMPUTE_F32 || dtype == KDA_F32;
  if (raw && f32c && dtype == KDA_BF16) return raw_unsupported("kda_segment_scan");
  int cus = 0;
  if (n_segments <= 0) {
    cus = kda_default_segments();
    if (cus < 0) return cus;
  }
  const int64_t req = n_segments > 0 ? n_segments : cus;  // the fused path's count
  hipStream_t st = (hipStream_t)stream;
  if (T > 0 && !f32c) {
    // two-kernel path: chunk prep over all chunks, segment pairs and the re-run
    // on the recurrence kernel; segments are ranges of chunk slots
    const SplitRequest sr = split_request(n_segments, H, cus);
    const SegPlan sp = plan_segments(used_chunk_slots(T, N, cu_seqlens_host), sr.n);
    if (sp.n_seg * H > kMaxSegHeads)
      return fail(KDA_ERR_SHAPE, "segments * H = %lld exceeds %lld (one launch)",
                  (long long)(sp.n_seg * H), (long long)kMaxSegHeads);
    const size_t need = split_scan_workspace(T, N, H, sr);
    if (!workspace || workspace_bytes < need)
      return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
    if (((uintptr_t)workspace & 255u) != 0) return fail(KDA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    // the buffers are laid out for the largest plan the workspace size allows for
    const int64_t n_max = max_split_segments(T, N, sr.n);
    const int64_t g_max = sr.one_level ? n_max : max_scan_groups(n_max);
    const int64_t glen = sr.one_level ? 1 : scan_group_len(sp.n_seg);
    const int64_t n_groups = (sp.n_seg + glen - 1) / glen;
    if (n_groups * H > kMaxGroupHeads)
      return fail(KDA_ERR_SHAPE, "segment groups * H = %lld exceeds %lld (one launch)",
                  (long long)(n_groups * H), (long long)kMaxGroupHeads);
    if (sp.n_seg > n_max || n_groups > g_max)
      return fail(KDA_ERR_UNSUPPORTED, "segment plan exceeds its workspace layout (%lld segments, %lld groups)",
                  (long long)sp.n_seg, (long long)n_groups);
    float *pairs = (float *)((char *)workspace + kda::split_workspace_bytes(T, N, H));
    float *gpairs = pairs + (size_t)n_max * H * kD * 2 * kD;
    float *gentry = gpairs + (size_t)g_max * H * kD * 2 * kD;

    kda::SplitParams p = split_params(q, k, v, g_logits, beta, A_log, g_min, initial_state,
                                      cu_seqlens, cu_seqlens_host, N, T, H, o, final_state,
                                      workspace);
    p.order = nullptr;  // segments, not documents
    p.n_seg = (int)sp.n_seg;
    p.seg_slots = sp.len;
    p.pairs = pairs;
    p.raw = raw;
    p.gate = gate;
    hipError_t e = kda::launch_chunk_prep(p, st);
    if (e != hipSuccess) return hip_fail(e, "kda_segment_scan prep");
    // Only the entry states of groups 1 .. n_groups - 1 come from pairs, so the
    // segments of the last group need none: pairs and their composition cover
    // the first n_groups - 1 groups.
    const int64_t paired = (n_groups - 1) * glen;  // < sp.n_seg
    if (paired > 0) {
      p.rmode = 2;  // A: segment pairs; resets at document starts are folded into them
      p.n_seg = (int)paired;
      e = kda::launch_chunk_recurrence(p, st);
      if (e != hipSuccess) return hip_fail(e, "kda_segment_scan pairs");
    }
    // B: entry states E_0 = 0, E_{j+1} = M_j E_j + S~_j (the first chunk is a
    // document start, so E_0 never matters), for the first segment of each
    // group of glen segments: the pairs of a group are composed into one, and
    // the group pairs are scanned
    const int n_cu = kda_default_segments();  // compute units, or an error status
    if (n_cu < 0) return n_cu;
    kda::ScanChains sc{};
    sc.H = H;
    if (paired > 0 && glen > 1) {
      sc.pairs = pairs;
      sc.n_pairs = (int)paired;
      sc.chain_len = (int)glen;
      sc.n_chains = (int)(n_groups - 1);
      sc.ncols = 2 * kD;
      sc.mode = 1;  // B1: compose each group of pairs
      sc.composed = gpairs;
      e = kda::launch_scan_chains(sc, n_cu, st);
      if (e != hipSuccess) return hip_fail(e, "kda_segment_scan group pairs");
    }
    // B2: entry state of each group (the last one after the last pair); groups
    // of one segment scan the segment pairs themselves
    sc.pairs = glen > 1 ? gpairs : pairs;
    sc.n_pairs = (int)(n_groups - 1);
    sc.chain_len = (int)n_groups;
    sc.n_chains = 1;
    sc.ncols = kD;
    sc.mode = 0;
    sc.write_final = 1;
    sc.states = gentry;
    e = kda::launch_scan_chains(sc, n_cu, st);
    if (e != hipSuccess) return hip_fail(e, "kda_segment_scan scan");
    // C: re-run the segments of each group back to back from the group's entry
    // state; each one then starts from the state the previous one ends with,
    // which is its exact entry state
    p.rmode = 1;
    p.n_seg = (int)n_groups;
    p.seg_slots = glen * sp.len;
    p.entry = gentry;
    e = kda::launch_chunk_recurrence(p, st);
    if (e != hipSuccess) return hip_fail(e, "kda_segment_scan re-run");
  } else if (T > 0) {
    const SegPlan sp = plan_segments(T, req);
    if (sp.n_seg * H > kMaxSegHeads)
      return fail(KDA_ERR_SHAPE, "segments * H = %lld exceeds %lld (one launch)",
                  (long long)(sp.n_seg * H), (long long)kMaxSegHeads);
    const size_t need = scan_workspace(sp.n_seg, H);
    if (!workspace || workspace_bytes < need)
      return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
    if (((uintptr_t)workspace & 255u) != 0) return fail(KDA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    float *pairs = (float *)workspace;
    float *entry = pairs + (size_t)sp.n_seg * H * kD * 2 * kD;
    const bool bf16_in = dtype == KDA_BF16;

    kda::FwdParams p{};
    p.q = q; p.k = k; p.v = v; p.z = g_logits; p.beta = beta;
    p.A_log = A_log; p.g_min = g_min;
    p.cu = cu_seqlens; p.N = N; p.T = T; p.H = H;
    p.n_items = (int)sp.n_seg; p.seg_len = sp.len;
    p.doc_init = initial_state;
    // A: segment pairs (M, S~)
    p.mode = 2; p.item_init = nullptr; p.o = nullptr; p.final_state = pairs;
    hipError_t e = kda::launch_fwd(p, bf16_in, f32c, gate, raw, st);
    if (e != hipSuccess) return hip_fail(e, "kda_segment_scan pairs");
    // B: entry states
    e = kda::launch_pair_scan(pairs, initial_state, cu_seqlens, N, H, (int)sp.n_seg, sp.len,
                              entry, st);
    if (e != hipSuccess) return hip_fail(e, "kda_segment_scan scan");
    // C: re-run every segment from its exact entry state
    p.mode = 1; p.item_init = entry; p.o = o; p.final_state = final_state;
    e = kda::launch_fwd(p, bf16_in, f32c, gate, raw, st);
    if (e != hipSuccess) return hip_fail(e, "kda_segment_scan re-run");
  }
  if (final_state && has_empty_doc(cu_seqlens_host, N, T)) {
    hipError_t e = kda::launch_copy_empty(cu_seqlens, T, initial_state, final_state, N, H, st);
    if (e != hipSuccess) return hip_fail(e, "kda_segment_scan empty documents");
  }
  return KDA_OK;
}

static int decode_common(float *state, int32_t S_pool, const int32_t *state_slots, const void *cq,
                         const void *ck, const void *cv, const void *cz, const void *cbeta,
                         const int32_t *accepted, int32_t W, const void *nq, const void *nk,
                         const void *nv, const void *nz, const void *nbeta,
                         const kda::DecodeWindowArgs &win, const float *A_log, float g_min,
                         void *o, int32_t *err_flag, int32_t N, int32_t H, int32_t dk,
                         int32_t dv, int32_t dtype, void *stream, const char *who) {
  const bool raw = take_raw_flag(dtype);
  const int gate = take_gate_flag(dtype);
  if (dk != kD || dv != kD) return fail(KDA_ERR_SHAPE, "only d_k = d_v = 128 is supported");
  if (N < 0 || H <= 0 || W < 0 || win.W2 < 0)
    return fail(KDA_ERR_SHAPE, "need N >= 0, H > 0, W >= 0, W2 >= 0");
  if (H > kMaxHeads) return fail(KDA_ERR_SHAPE, "H must be at most %d (got %d)", kMaxHeads, H);
  if ((int64_t)N * H > kMaxSeqHeads)
    return fail(KDA_ERR_SHAPE, "N * H = %lld exceeds %lld (one launch)", (long long)N * H,
                (long long)kMaxSeqHeads);
  if (dtype != KDA_F32 && dtype != KDA_BF16) return fail(KDA_ERR_DTYPE, "unknown dtype %d", dtype);
  if (gate == kda::GATE_BOUNDED && !(g_min >= -5.0f && g_min < 0.0f))
    return fail(KDA_ERR_GATE_BOUND, "g_min must lie in [-5, 0) (got %g)", (double)g_min);
  if (S_pool < 0) return fail(KDA_ERR_SHAPE, "S_pool must be >= 0 (got %d)", S_pool);
  if (!state_slots && S_pool < N)
    return fail(KDA_ERR_SHAPE, "without state_slots the pool needs N = %d states (S_pool = %d)", N, S_pool);
  if ((int64_t)S_pool * H > (int64_t)INT32_MAX) return fail(KDA_ERR_SHAPE, "S_pool * H too large");
  if (N == 0) return KDA_OK;
  if (!state || !accepted || !nq || !nk || !nv || !nz || !nbeta || !o)
    return fail(KDA_ERR_NULL, "state, accepted, bonus inputs and o must be non-NULL");
  if (W > 0 && (!cq || !ck || !cv || !cz || !cbeta))
    return fail(KDA_ERR_NULL, "draft caches must be non-NULL when W > 0");
  if (win.W2 > 0 && (!win.q || !win.k || !win.v || !win.z || !win.beta || !win.o))
    return fail(KDA_ERR_NULL, "next-window inputs and outputs must be non-NULL when W2 > 0");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = (dtype == KDA_BF16)
      ? kda::launch_decode<kda::bf16_t>(state, state_slots, cq, ck, cv, cz, cbeta, accepted, W, nq,
                                        nk, nv, nz, nbeta, win, raw, A_log, g_min, gate, o,
                                        err_flag, N, H, S_pool, st)
      : kda::launch_decode<float>(state, state_slots, cq, ck, cv, cz, cbeta, accepted, W, nq, nk,
                                  nv, nz, nbeta, win, raw, A_log, g_min, gate, o, err_flag, N,
                                  H, S_pool, st);
  if (e != hipSuccess) return hip_fail(e, who);
  return KDA_OK;
}

int kda_decode_step(float *state, int32_t S_pool, const int32_t *state_slots, const void *cq,
                    const void *ck,
                    const void *cv, const void *cz, const void *cbeta,
                    const int32_t *accepted, int32_t W, const void *nq, const void *nk,
                    const void *nv, const void *nz, const void *nbeta, const float *A_log,
                    float g_min, void *o, int32_t *err_flag, int32_t N, int32_t H, int32_t dk,
                    int32_t dv, int32_t dtype, void *stream) {
  const kda::DecodeWindowArgs none{0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  return decode_common(state, S_pool, state_slots, cq, ck, cv, cz, cbeta, accepted, W, nq, nk, nv,
                       nz, nbeta, none, A_log, g_min, o, err_flag, N, H, dk, dv, dtype, stream,
                       "kda_decode_step launch");
}

int kda_decode_step_window(float *state, int32_t S_pool, const int32_t *state_slots,
                           const void *cq,
                           const void *ck, const void *cv, const void *cz, const void *cbeta,
                           const int32_t *accepted, int32_t W, const void *nq, const void *nk,
                           const void *nv, const void *nz, const void *nbeta, const void *wq,
                           const void *wk, const void *wv, const void *wz, const void *wbeta,
                           int32_t W2, const float *A_log, float g_min, void *o, void *o_window,
                           int32_t *err_flag, int32_t N, int32_t H, int32_t dk, int32_t dv,
                           int32_t dtype, void *stream) {
  const kda::DecodeWindowArgs win{W2, wq, wk, wv, wz, wbeta, o_window};
  return decode_common(state, S_pool, state_slots, cq, ck, cv, cz, cbeta, accepted, W, nq, nk, nv,
                       nz, nbeta, win, A_log, g_min, o, err_flag, N, H, dk, dv, dtype, stream,
                       "kda_decode_step_window launch");
}

}  // extern "C"
