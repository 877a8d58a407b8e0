// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace attn_sink {

constexpr int kHeadDimBuilt = 64;  // the only head dim the kernels are built for

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
};

struct BwdArgs {
  FwdArgs f;        // q, k, v, sinks, cu_*, shape; f.o / f.lse are the forward outputs (read-only)
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* dsinks;
  // workspace carve-up (float32, device)
  float* rowstat;     // [hq, 2, total_q]: lse_i * log2(e), then -D_i with D_i = <dO_i, O_i>
  float* dsink_part;  // [hq, pre_blocks]
  float* dk_part;     // [splits, total_k, hkv, 64] (only when splits > 1)
  float* dv_part;     // [splits, total_k, hkv, 64] (only when splits > 1)
  int pre_blocks;
  int splits;         // workgroups sharing one kv head's query-head group in bwd_dkdv
};

// Kernel identifiers for the opt-in timing records.
enum KernelId { K_FWD = 0, K_BWD_PRE = 1, K_BWD_DQ = 2, K_BWD_DKDV = 3, K_BWD_FINISH = 4, K_COUNT = 5 };
const char* kernel_name(int id);

// Workspace layout for a backward call; offsets in bytes from the workspace base.
struct BwdWorkspace {
  size_t rowstat, dsink_part, dk_part, dv_part, total;
  int pre_blocks, splits;
};
BwdWorkspace bwd_workspace_layout(int hq, int hkv, int total_q, int total_k, int num_seqs);
int bwd_head_splits(int hq, int hkv, int total_k, int num_seqs);

// Each launcher enqueues one kernel on `stream` and returns hipGetLastError().
hipError_t launch_fwd(const FwdArgs& a, int fp32, hipStream_t stream);
hipError_t launch_bwd_pre(const BwdArgs& a, int fp32, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, int fp32, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, int fp32, hipStream_t stream);
hipError_t launch_bwd_finish(const BwdArgs& a, int fp32, hipStream_t stream);

}  // namespace attn_sink
