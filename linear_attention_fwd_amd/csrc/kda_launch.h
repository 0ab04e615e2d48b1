// kda_launch.h -- host-side launchers of the KDA kernels (internal to libkda.so).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef uint16_t bf16_t;  // storage type of bf16 tensors

struct FwdParams {
  const void *q, *k, *v, *z, *beta;
  const float *A_log;
  float g_min;
  const int32_t *cu;       // [N+1] device document offsets, or nullptr = one document [0, T)
  int N;
  int64_t T;
  int H;
  int mode;                // 0: items are documents; 1: items are seg_len-token segments
                           // (re-run from entry states); 2: segment pairs (M, S~)
  int n_items;
  int64_t seg_len;
  const float *item_init;  // mode 0: initial state per document (or nullptr = 0);
                           // mode 1: entry state per segment [n_items, H, D, D]
  const float *doc_init;   // modes 1, 2: initial state per document (or nullptr = 0)
  void *o;                 // mode 0, 1: output [T, H, D]
  float *final_state;      // modes 0, 1: [N, H, D, D] or nullptr; mode 2: pairs
                           // [n_items, H, D, 2D] (columns 0..127 = S~, 128..255 = M)
  int nsplit;              // set by the launcher
};
constexpr int GATE_BOUNDED = 0, GATE_SOFTPLUS = 1;

// gate: GATE_BOUNDED or GATE_SOFTPLUS (the unbounded gate, g_min unused); raw:
// q, k L2-normalised and the beta sigmoid in the kernel.  Raw inputs with bf16
// inputs and fp32 arithmetic are not supported (the normalised rows would be
// rounded to bf16); the caller refuses them.
hipError_t launch_fwd(FwdParams p, bool bf16_in, bool f32_compute, int gate, bool raw,
                      hipStream_t stream);

// Chunk slots: chunk k of document d (chunks of 64 tokens restart at every
// document start) lives in slot  first_slot(cu[d], d) + k  with
// first_slot = floor(cu[d] / 64) + d.  The map is injective and needs no prefix
// sum over documents; every slot lies in [0, n_chunk_slots(T, N)), and slots no
// chunk maps to are skipped.
__host__ __device__ inline int64_t first_slot(int64_t cu_d, int d) { return cu_d / 64 + d; }
__host__ __device__ inline int64_t n_chunk_slots(int64_t T, int N) { return T / 64 + N; }

// Two-kernel prefill over documents (bf16 inputs, bf16 MFMA operands): a
// token-parallel prep kernel writes every (head, chunk) "chunk image" (the
// recurrence operands, laid out as the recurrence kernel's LDS tiles) into the
// workspace, then the recurrence kernel streams the images of each document
// through double-buffered LDS.
struct SplitParams {
  const void *q, *k, *v, *z, *beta;
  const float *A_log;
  float g_min;
  const int32_t *cu;       // [N+1] device document offsets, or nullptr = one document [0, T)
  int N;
  int64_t T;
  int H;
  const float *init;       // [N, H, D, D] initial states or nullptr (= 0)
  void *o;                 // [T, H, D]
  float *final_state;      // [N, H, D, D] or nullptr
  void *ws;                // chunk images [H, n_slots, image]
  int64_t n_slots;         // chunk slots per head (see first_slot)
  // recurrence work split: 0 = one item per document; 1 = segment re-run from
  // entry states; 2 = segment pairs (M, S~).  Segments are ranges of seg_slots
  // chunk slots.
  int rmode;
  int n_seg;
  int64_t seg_slots;
  const float *entry;      // mode 1: entry state per segment [n_seg, H, D, D]
  float *pairs;            // mode 2: [n_seg, H, D, 2D], columns 0..127 S~, 128..255 M
  // modes 0 and 1: the state after every ckpt_chunks-th chunk of a document
  // (not after its last chunk) to ckpt[slot / ckpt_chunks, H, D, D]; 0 = none
  float *ckpt;
  int ckpt_chunks;
  // gate map: GATE_BOUNDED (g_min * sigmoid) or GATE_SOFTPLUS (unbounded,
  // g_min unused); only the prep kernel depends on it
  int gate;
  // raw inputs: the prep kernel L2-normalises q and k and applies the sigmoid
  // to beta
  int raw;
  // mode 0: the order in which the recurrence takes the documents (longest
  // first), [N] in the workspace after the images, written by launch_chunk_prep;
  // nullptr = input order
  int32_t *order;
};
// Bytes of one chunk image (the recurrence operands of one (head, chunk);
// the layout is ChunkImage in kda_split.hip, which checks this size).
constexpr int64_t CHUNK_IMAGE_BYTES = 62464;
// chunk images [H, n_slots, image], then the document order (4 N bytes,
// rounded up to 256)
inline size_t split_order_offset(int64_t T, int N, int H) {
  return (size_t)n_chunk_slots(T, N) * (size_t)H * (size_t)CHUNK_IMAGE_BYTES;
}
inline size_t split_workspace_bytes(int64_t T, int N, int H) {
  return split_order_offset(T, N, H) + ((size_t)N * 4 + 255) / 256 * 256;
}
hipError_t launch_chunk_prep(const SplitParams &p, hipStream_t stream);
// Device scratch of kda_chunk_fwd_noalloc (kda_noalloc.hip): the address, on the
// current device, of a static array of NOALLOC_SCRATCH_BYTES bytes.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)256 << 20;
hipError_t noalloc_scratch(void **ptr);
hipError_t launch_chunk_recurrence(const SplitParams &p, hipStream_t stream);

// final_state[d] = initial_state[d] (or 0) for every empty document d;
// cu == nullptr means one document of T tokens.
hipError_t launch_copy_empty(const int32_t *cu, int64_t T, const float *init, float *fin, int N,
                             int H, hipStream_t stream);
hipError_t launch_pair_scan(const float *pairs, const float *S0, const int32_t *cu, int N,
                            int H, int n_seg, int64_t seg_len, float *entry, hipStream_t stream);

// Chains of segment-pair applications (a scan of pairs in levels); see
// kda_scan_chains_kernel.  Pairs are [n_pairs, H, D, 2D] (columns 0..127 S~,
// 128..255 M); chain c covers pairs [c * chain_len, min((c + 1) * chain_len, n_pairs)).
struct ScanChains {
  const float *pairs;
  int H;
  int n_pairs;
  int chain_len;
  int n_chains;
  int ncols;          // 128 (states) or 256 (compose)
  int mode;           // 0: write the state before each pair to states[i]; 1: compose
  int write_final;    // mode 0: also write the state after a chain's last pair to states[last]
  const float *init;  // mode 0: [n_chains, H, D, D] chain start states, or nullptr (0)
  float *states;      // mode 0: [n_pairs, H, D, D]
  float *composed;    // mode 1: [n_chains, H, D, 2D]
};
// n_cu: compute units of the device (chooses the columns per workgroup)
hipError_t launch_scan_chains(const ScanChains &sc, int n_cu, hipStream_t stream);

// Drafts of the next window that a decode step runs after the bonus token
// (outputs only): q, k, v, z [N, W2, H, D], beta [N, W2, H], o [N, W2, H, D];
// W2 = 0 and null pointers when there is no window.
struct DecodeWindowArgs {
  int W2;
  const void *q, *k, *v, *z, *beta;
  void *o;
};

template <typename Tin>
hipError_t launch_decode(float *state, const int32_t *slots, const void *cq, const void *ck,
                         const void *cv, const void *cz, const void *cbeta,
                         const int32_t *accepted, int W, const void *nq, const void *nk,
                         const void *nv, const void *nz, const void *nbeta,
                         const DecodeWindowArgs &win, bool raw, const float *A_log,
                         float g_min, int gate, void *o, int32_t *err_flag, int N, int H,
                         int S_pool, hipStream_t stream);

}  // namespace kda
