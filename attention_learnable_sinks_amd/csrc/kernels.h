// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace attn_sink {

// Head dims the kernels are built for.
inline bool head_dim_built(int d) { return d == 64 || d == 128; }

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* sinks;
  void* o;
  float* lse;
  const int* cu_q;
  const int* cu_k;
  int hq, hkv, num_seqs, total_q, total_k, max_q, max_k;
  float scale;
  int causal, window;
  int d;  // head dim: 64 or 128
};

struct BwdArgs {
  FwdArgs f;        // q, k, v, sinks, cu_*, shape; f.o / f.lse are the forward outputs (read-only)
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* dsinks;
  // workspace carve-up (float32, device)
  float* rowstat;     // [hq, 2, total_q]: lse_i * log2(e), then -D_i with D_i = <dO_i, O_i> (written by bwd_dq)
  float* dsink_part;  // [hq, pre_blocks]: per (sequence, dQ row tile) partial sums of -P_sink_i D_i
  float* dk_part;     // [splits, total_k, hkv, 64] (only when splits > 1)
  float* dv_part;     // [splits, total_k, hkv, 64] (only when splits > 1)
  int pre_blocks;
  int splits;         // workgroups sharing one kv head's query-head group in bwd_dkdv
};

// Forward for a few query rows per sequence against long key ranges, split over keys.
struct DecodeArgs {
  FwdArgs f;
  float* part_o;   // [num_seqs * hkv, max_chunks, cols, d]: unnormalised O of each key chunk
  float* part_ml;  // [num_seqs * hkv, max_chunks, cols, 2]: (running max, sum) in the exp2 domain
  int chunk;       // key tiles (of 64) per chunk
  int max_chunks;  // chunks of the longest visible key range (grid y)
  int cols;        // (Hq / Hkv) * max_seqlen_q: columns per (sequence, kv head)
  int hw;          // kv heads (wavefronts) per workgroup
};

// Merge of per-shard attention partials (no sink) into the sink attention output.
struct MergeArgs {
  const void* o_parts;     // [parts, total_q, hq, 64], element type of the call
  const float* lse_parts;  // [parts, hq, total_q], natural log, no sink
  const float* sinks;      // [hq]
  void* o;                 // [total_q, hq, 64]
  float* lse;              // [hq, total_q], sink included
  int parts, hq, total_q, d;
};

// Kernel identifiers for the opt-in timing records.
enum KernelId {
  K_FWD = 0, K_BWD_DQ = 1, K_BWD_DKDV = 2, K_BWD_FINISH = 3,
  K_DEC_PARTIAL = 4, K_DEC_MERGE = 5, K_MERGE = 6, K_COUNT = 7
};
const char* kernel_name(int id);

// Tile shapes the host-side layout shares with the kernels (static_assert'ed there).
constexpr int kDqRows = 128;      // query rows per dQ workgroup
constexpr int kDkvKeys = 128;     // keys per dK/dV workgroup tile
constexpr int kDecodeKeys = 32;   // keys per decoding tile
constexpr int kDecodeCols = 32;   // (query head, row) columns per kv head in the decoding kernels
constexpr int kDecodeWaves = 4;   // kv heads (wavefronts) per decoding workgroup at most
constexpr int kDecodeChunk = 32;  // key tiles per decoding chunk (1024 keys)

// Head-packed dQ tiles (window layers) and dQ row tiles per sequence.
bool dq_head_packed(int hq, int hkv, int num_seqs, int max_q, int window);
// Head-packed dK/dV query tiles (window layers, bf16, 8 query heads per kv head, one split).
inline bool dkdv_head_packed(int hq, int hkv, int window, int splits) {
  return window > 0 && splits == 1 && hkv > 0 && hq == 8 * hkv;
}
int dq_tiles(int hq, int hkv, int num_seqs, int max_q, int window);

// Workspace layout for a backward call; offsets in bytes from the workspace base.
struct BwdWorkspace {
  size_t rowstat, dsink_part, dk_part, dv_part, total;
  int pre_blocks, splits;
};
BwdWorkspace bwd_workspace_layout(int hq, int hkv, int total_q, int total_k, int num_seqs, int max_q, int causal,
                                  int window, int d, int fp32);
int bwd_head_splits(int hq, int hkv, int total_k, int num_seqs, int causal, int window, int d, int fp32);

struct DecodeWorkspace {
  size_t part_o, part_ml, total;
  int chunk, max_chunks, cols, hw;
};
DecodeWorkspace decode_workspace_layout(int fp32, int hq, int hkv, int num_seqs, int max_q, int max_k, int window,
                                        int d);
// The query heads of one kv head times the rows of one sequence fill at most 32 columns.
bool decode_supported(int hq, int hkv, int max_q);

// Size of the decoding forward's fixed scratch (one static device array per GPU) and
// its address on the current device (looked up on the device's first call, then kept).
constexpr size_t kDecodeScratchBytes = (size_t)64 << 20;
hipError_t decode_scratch(void** ptr);

// Each launcher enqueues one kernel on `stream` and returns hipGetLastError().
hipError_t launch_fwd(const FwdArgs& a, int fp32, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, int fp32, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, int fp32, hipStream_t stream);
hipError_t launch_bwd_finish(const BwdArgs& a, int fp32, hipStream_t stream);
hipError_t launch_decode_partial(const DecodeArgs& a, int fp32, hipStream_t stream);
hipError_t launch_decode_merge(const DecodeArgs& a, int fp32, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, int fp32, hipStream_t stream);

}  // namespace attn_sink
