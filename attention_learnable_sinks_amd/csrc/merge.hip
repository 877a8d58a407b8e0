// Merge of attention partials computed over disjoint key shards, with the per-head
// sink counted exactly once (context / sequence parallelism across devices, where
// each device attends its query rows to one shard of the keys at a time).
//
// Each part s holds, per query row i and head h, the standard-attention output over
// its shard's keys, O_s = sum_{j in s} exp(s_ij - LSE_s) v_j, and LSE_s =
// log sum_{j in s} exp(s_ij) (no sink; -inf where the row sees no key of the shard).
// The sink joins the normaliser once ("Unlocking Agentic RL Training for GPT-OSS",
// 数学公式: one extra exp(S_h) in the denominator, never multiplied by V):
//   M   = max(S_h, max_s LSE_s)
//   L   = exp(S_h - M) + sum_s exp(LSE_s - M)
//   o_i = sum_s exp(LSE_s - M) O_s / L,     lse_i = M + log L
// Parts are folded in index order, so the result is bitwise repeatable.
#include "common.h"
#include "kernels.h"

namespace attn_sink {

// One wavefront per (row, head), lane = d (and d + 64 when D = 128); 4 per workgroup.
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  constexpr int DL = D / 64;  // values of d per lane
  const long long pair = (long long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long long pairs = (long long)a.total_q * a.hq;
  if (pair >= pairs) return;
  const int row = (int)(pair / a.hq), head = (int)(pair % a.hq);
  const int d = threadIdx.x & 63;
  const size_t lse_at = (size_t)head * a.total_q + row;       // [part][Hq][total_q]
  const size_t o_at = ((size_t)row * a.hq + head) * D + d;    // [part][total_q][Hq][D]
  const size_t lse_stride = (size_t)a.hq * a.total_q, o_stride = (size_t)a.total_q * a.hq * D;
  const T* o_parts = static_cast<const T*>(a.o_parts);
  const float sink = a.sinks[head];
  constexpr int U = 8;
  float mm = sink;
  for (int s0 = 0; s0 < a.parts; s0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (s0 + u < a.parts) mm = fmaxf(mm, a.lse_parts[(size_t)(s0 + u) * lse_stride + lse_at]);
  }
  float o[DL], l = 0.f;
#pragma unroll
  for (int j = 0; j < DL; ++j) o[j] = 0.f;
  if (mm > -INFINITY) {
    l = sink > -INFINITY ? __expf(sink - mm) : 0.f;  // the sink's mass, once
    for (int s0 = 0; s0 < a.parts; s0 += U) {
      float ls[U], os[U][DL];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool ok = s0 + u < a.parts;
        ls[u] = ok ? a.lse_parts[(size_t)(s0 + u) * lse_stride + lse_at] : -INFINITY;
#pragma unroll
        for (int j = 0; j < DL; ++j) os[u][j] = ok ? to_f32(o_parts[(size_t)(s0 + u) * o_stride + o_at + 64 * j]) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float w = ls[u] == -INFINITY ? 0.f : __expf(ls[u] - mm);  // a shard the row does not see
        l += w;
#pragma unroll
        for (int j = 0; j < DL; ++j) o[j] += w * os[u][j];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < DL; ++j)
    static_cast<T*>(a.o)[((size_t)row * a.hq + head) * D + d + 64 * j] = from_f32<T>(l > 0.f ? o[j] / l : 0.f);
  if (d == 0) a.lse[lse_at] = l > 0.f ? mm + __logf(l) : -INFINITY;
}

hipError_t launch_merge(const MergeArgs& a, int fp32, hipStream_t stream) {
  const long long pairs = (long long)a.total_q * a.hq;
  if (pairs == 0) return hipSuccess;
  dim3 grid((unsigned)((pairs + 3) / 4));
  if (a.d == 128) {
    if (fp32)
      hipLaunchKernelGGL((merge_kernel<float, 128>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((merge_kernel<bf16, 128>), grid, dim3(256), 0, stream, a);
  } else {
    if (fp32)
      hipLaunchKernelGGL((merge_kernel<float, 64>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((merge_kernel<bf16, 64>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace attn_sink
