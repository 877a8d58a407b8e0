// C ABI of the attention-with-sinks library: argument checks, workspace carve-up,
// kernel launches and the opt-in per-kernel timing records.  The operations are
// defined in include/attn_sink.h.
#include "attn_sink.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <initializer_list>
#include <mutex>
#include <vector>

#include "kernels.h"

namespace attn_sink {

const char* kernel_name(int id) {
  switch (id) {
    case K_FWD: return "attn_sink_fwd_kernel";
    case K_BWD_DQ: return "attn_sink_bwd_dq_kernel";
    case K_BWD_DKDV: return "attn_sink_bwd_dkdv_kernel";
    case K_BWD_FINISH: return "attn_sink_bwd_finish_kernel";
    case K_DEC_PARTIAL: return "attn_sink_decode_partial_kernel";
    case K_DEC_MERGE: return "attn_sink_decode_merge_kernel";
    case K_MERGE: return "attn_sink_merge_kernel";
    default: return "?";
  }
}

namespace {

// ---- opt-in timing records: the library's only mutable host state.  With timing
// off (the default) a launch reads the flag and nothing else; with it on, each
// launch appends one event pair under the mutex.
struct Record {
  int kernel;
  hipEvent_t start, stop;
};
std::mutex g_mu;  // guards g_records
std::atomic<bool> g_timing{false};
std::vector<Record> g_records;

void clear_records_locked() {
  for (auto& r : g_records) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_records.clear();
}

template <typename F>
attn_sink_status timed_launch(int kernel, hipStream_t stream, F&& launch) {
  const bool timing = g_timing.load(std::memory_order_acquire);
  Record rec{kernel, nullptr, nullptr};
  // Events of a failed launch are released here (a recorded event may be destroyed
  // before it completes; the runtime frees it once it has).
  auto fail = [&rec]() {
    if (rec.start) (void)hipEventDestroy(rec.start);
    if (rec.stop) (void)hipEventDestroy(rec.stop);
    return ATTN_SINK_ERR_HIP;
  };
  if (timing) {
    if (hipEventCreate(&rec.start) != hipSuccess) return fail();
    if (hipEventCreate(&rec.stop) != hipSuccess) return fail();
    if (hipEventRecord(rec.start, stream) != hipSuccess) return fail();
  }
  if (launch() != hipSuccess) return fail();
  if (timing) {
    if (hipEventRecord(rec.stop, stream) != hipSuccess) return fail();
    std::lock_guard<std::mutex> lk(g_mu);
    g_records.push_back(rec);
  }
  return ATTN_SINK_OK;
}

// Tensor pointers the kernels access in 16-byte pieces, and 4-byte scalar arrays.
// A null pointer passes here; the null checks of each entry point come first.
bool misaligned(std::initializer_list<const void*> wide, std::initializer_list<const void*> narrow) {
  for (const void* p : wide)
    if (reinterpret_cast<uintptr_t>(p) & 15) return true;
  for (const void* p : narrow)
    if (reinterpret_cast<uintptr_t>(p) & 3) return true;
  return false;
}

attn_sink_status check_shape(const attn_sink_shape* s) {
  if (!s) return ATTN_SINK_ERR_INVALID_ARG;
  if (s->dtype != ATTN_SINK_BF16 && s->dtype != ATTN_SINK_FP32) return ATTN_SINK_ERR_UNSUPPORTED;
  if (!head_dim_built(s->head_dim)) return s->head_dim > 0 ? ATTN_SINK_ERR_UNSUPPORTED : ATTN_SINK_ERR_INVALID_ARG;
  if (s->num_heads_q < 1 || s->num_heads_kv < 1 || s->num_heads_q % s->num_heads_kv != 0)
    return ATTN_SINK_ERR_INVALID_ARG;
  if (s->num_seqs < 1 || s->total_q < 0 || s->total_k < 0 || s->max_seqlen_q < 0 || s->max_seqlen_k < 0)
    return ATTN_SINK_ERR_INVALID_ARG;
  if (!s->cu_seqlens_q || !s->cu_seqlens_k) return ATTN_SINK_ERR_INVALID_ARG;
  if (misaligned({}, {s->cu_seqlens_q, s->cu_seqlens_k})) return ATTN_SINK_ERR_INVALID_ARG;
  if (!(s->softmax_scale > 0.f) || !std::isfinite(s->softmax_scale)) return ATTN_SINK_ERR_INVALID_ARG;
  if (s->causal != 0 && s->causal != 1) return ATTN_SINK_ERR_INVALID_ARG;
  // grid limits: y is the tile index (<= 65535); x is heads * sequences
  if ((long long)s->num_heads_q * s->num_seqs > 0x7fffffffLL) return ATTN_SINK_ERR_UNSUPPORTED;
  if (s->max_seqlen_q > 65535LL * 128 || s->max_seqlen_k > 65535LL * 128) return ATTN_SINK_ERR_UNSUPPORTED;
  // Each kernel reads one head of one sequence through a buffer descriptor with
  // 32-bit byte offsets; a tile (at most 128 rows) may start on the last row, so
  // (rows + 128) x row pitch must fit in 32 bits.
  const long long esize = s->dtype == ATTN_SINK_FP32 ? 4 : 2;
  if ((s->max_seqlen_q + 128LL) * s->num_heads_q * s->head_dim * esize >= (1LL << 32) ||
      (s->max_seqlen_k + 128LL) * s->num_heads_kv * s->head_dim * esize >= (1LL << 32))
    return ATTN_SINK_ERR_UNSUPPORTED;
  // 32-bit row indices inside the kernels
  if ((long long)s->total_q * s->num_heads_q * s->head_dim > 0x7fffffffLL * 4LL) return ATTN_SINK_ERR_UNSUPPORTED;
  return ATTN_SINK_OK;
}

FwdArgs fwd_args(const attn_sink_shape* s, const void* q, const void* k, const void* v, const float* sinks,
                 const void* o, const float* lse) {
  FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.sinks = sinks;
  a.o = const_cast<void*>(o);
  a.lse = const_cast<float*>(lse);
  a.cu_q = s->cu_seqlens_q;
  a.cu_k = s->cu_seqlens_k;
  a.hq = s->num_heads_q;
  a.hkv = s->num_heads_kv;
  a.num_seqs = s->num_seqs;
  a.total_q = s->total_q;
  a.total_k = s->total_k;
  a.max_q = s->max_seqlen_q;
  a.max_k = s->max_seqlen_k;
  a.scale = s->softmax_scale;
  a.causal = s->causal;
  a.window = s->window > 0 ? s->window : 0;
  a.d = s->head_dim;
  return a;
}

DecodeWorkspace decode_layout(const attn_sink_shape* s) {
  return decode_workspace_layout(s->dtype == ATTN_SINK_FP32, s->num_heads_q, s->num_heads_kv, s->num_seqs,
                                 s->max_seqlen_q, s->max_seqlen_k, s->window > 0 ? s->window : 0, s->head_dim);
}

// Checks shared by the two decoding entry points; fills `ws`.
attn_sink_status decode_checks(const attn_sink_shape* shape, const void* q, const void* k, const void* v,
                               const float* sinks, void* o, float* lse, DecodeWorkspace* ws) {
  attn_sink_status st = check_shape(shape);
  if (st != ATTN_SINK_OK) return st;
  if (!decode_supported(shape->num_heads_q, shape->num_heads_kv, shape->max_seqlen_q)) return ATTN_SINK_ERR_UNSUPPORTED;
  const bool any_q = shape->total_q > 0, any_k = shape->total_k > 0;
  if (!sinks || (any_q && (!q || !o || !lse)) || (any_k && (!k || !v))) return ATTN_SINK_ERR_INVALID_ARG;
  if (misaligned({q, k, v, o}, {sinks, lse})) return ATTN_SINK_ERR_INVALID_ARG;
  *ws = decode_layout(shape);
  return ATTN_SINK_OK;
}

DecodeArgs decode_args(const attn_sink_shape* shape, const void* q, const void* k, const void* v,
                       const float* sinks, void* o, float* lse, const DecodeWorkspace& ws, void* workspace) {
  DecodeArgs a;
  a.f = fwd_args(shape, q, k, v, sinks, o, lse);
  char* base = static_cast<char*>(workspace);
  a.part_o = reinterpret_cast<float*>(base + ws.part_o);
  a.part_ml = reinterpret_cast<float*>(base + ws.part_ml);
  a.chunk = ws.chunk;
  a.max_chunks = ws.max_chunks;
  a.cols = ws.cols;
  a.hw = ws.hw;
  return a;
}

}  // namespace
}  // namespace attn_sink

using namespace attn_sink;

extern "C" {

attn_sink_status attn_sink_fwd(const attn_sink_shape* shape, const void* q, const void* k, const void* v,
                               const float* sinks, void* o, float* lse, hipStream_t stream) {
  attn_sink_status st = check_shape(shape);
  if (st != ATTN_SINK_OK) return st;
  const bool any_q = shape->total_q > 0, any_k = shape->total_k > 0;
  if (!sinks || (any_q && (!q || !o || !lse)) || (any_k && (!k || !v))) return ATTN_SINK_ERR_INVALID_ARG;
  if (misaligned({q, k, v, o}, {sinks, lse})) return ATTN_SINK_ERR_INVALID_ARG;
  if (!any_q) return ATTN_SINK_OK;
  FwdArgs a = fwd_args(shape, q, k, v, sinks, o, lse);
  const int fp32 = shape->dtype == ATTN_SINK_FP32;
  return timed_launch(K_FWD, stream, [&] { return launch_fwd(a, fp32, stream); });
}

size_t attn_sink_fwd_decode_workspace_bytes(const attn_sink_shape* shape) {
  if (check_shape(shape) != ATTN_SINK_OK) return 0;
  if (!decode_supported(shape->num_heads_q, shape->num_heads_kv, shape->max_seqlen_q)) return 0;
  return decode_layout(shape).total;
}

attn_sink_status attn_sink_fwd_decode(const attn_sink_shape* shape, const void* q, const void* k, const void* v,
                                      const float* sinks, void* o, float* lse, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  DecodeWorkspace ws;
  attn_sink_status st = decode_checks(shape, q, k, v, sinks, o, lse, &ws);
  if (st != ATTN_SINK_OK) return st;
  if (!workspace || workspace_bytes < ws.total || (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return ATTN_SINK_ERR_WORKSPACE;
  if (shape->total_q == 0) return ATTN_SINK_OK;
  const DecodeArgs a = decode_args(shape, q, k, v, sinks, o, lse, ws, workspace);
  const int fp32 = shape->dtype == ATTN_SINK_FP32;
  st = timed_launch(K_DEC_PARTIAL, stream, [&] { return launch_decode_partial(a, fp32, stream); });
  if (st != ATTN_SINK_OK || ws.max_chunks <= 1) return st;  // one chunk: finished in place
  return timed_launch(K_DEC_MERGE, stream, [&] { return launch_decode_merge(a, fp32, stream); });
}

attn_sink_status attn_sink_fwd_decode_noalloc(const attn_sink_shape* shape, const void* q, const void* k,
                                              const void* v, const float* sinks, void* o, float* lse,
                                              hipStream_t stream) {
  DecodeWorkspace ws;
  attn_sink_status st = decode_checks(shape, q, k, v, sinks, o, lse, &ws);
  if (st != ATTN_SINK_OK) return st;
  if (ws.total > kDecodeScratchBytes) return ATTN_SINK_ERR_WORKSPACE;  // beyond the fixed scratch
  // The scratch used is the current device's copy, so the stream must belong to it.
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_SINK_ERR_HIP;
  if (stream != nullptr) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return ATTN_SINK_ERR_HIP;
    if (sdev != dev) return ATTN_SINK_ERR_INVALID_ARG;
  }
  void* base = nullptr;
  if (decode_scratch(&base) != hipSuccess) return ATTN_SINK_ERR_HIP;
  if (shape->total_q == 0) return ATTN_SINK_OK;
  const DecodeArgs a = decode_args(shape, q, k, v, sinks, o, lse, ws, base);
  const int fp32 = shape->dtype == ATTN_SINK_FP32;
  // Launched without the timing records (their events would be created here).
  if (launch_decode_partial(a, fp32, stream) != hipSuccess) return ATTN_SINK_ERR_HIP;
  if (ws.max_chunks <= 1) return ATTN_SINK_OK;  // one chunk: finished in place
  return launch_decode_merge(a, fp32, stream) == hipSuccess ? ATTN_SINK_OK : ATTN_SINK_ERR_HIP;
}

size_t attn_sink_bwd_workspace_bytes(const attn_sink_shape* shape) {
  if (check_shape(shape) != ATTN_SINK_OK) return 0;
  return bwd_workspace_layout(shape->num_heads_q, shape->num_heads_kv, shape->total_q, shape->total_k, shape->num_seqs,
                              shape->max_seqlen_q, shape->causal, shape->window > 0 ? shape->window : 0,
                              shape->head_dim, shape->dtype == ATTN_SINK_FP32).total;
}

attn_sink_status attn_sink_bwd(const attn_sink_shape* shape, const void* q, const void* k, const void* v,
                               const float* sinks, const void* o, const float* lse, const void* dout, void* dq,
                               void* dk, void* dv, float* dsinks, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  attn_sink_status st = check_shape(shape);
  if (st != ATTN_SINK_OK) return st;
  const bool any_q = shape->total_q > 0, any_k = shape->total_k > 0;
  if (!sinks || !dsinks) return ATTN_SINK_ERR_INVALID_ARG;
  if (any_q && (!q || !o || !lse || !dout || !dq)) return ATTN_SINK_ERR_INVALID_ARG;
  if (any_k && (!k || !v || !dk || !dv)) return ATTN_SINK_ERR_INVALID_ARG;
  if (misaligned({q, k, v, o, dout, dq, dk, dv}, {sinks, lse, dsinks})) return ATTN_SINK_ERR_INVALID_ARG;
  const BwdWorkspace ws = bwd_workspace_layout(shape->num_heads_q, shape->num_heads_kv, shape->total_q, shape->total_k, shape->num_seqs,
                              shape->max_seqlen_q, shape->causal, shape->window > 0 ? shape->window : 0,
                              shape->head_dim, shape->dtype == ATTN_SINK_FP32);
  if (!workspace || workspace_bytes < ws.total || (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return ATTN_SINK_ERR_WORKSPACE;

  BwdArgs a;
  a.f = fwd_args(shape, q, k, v, sinks, o, lse);
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dsinks = dsinks;
  char* base = static_cast<char*>(workspace);
  a.rowstat = reinterpret_cast<float*>(base + ws.rowstat);
  a.dsink_part = reinterpret_cast<float*>(base + ws.dsink_part);
  a.dk_part = reinterpret_cast<float*>(base + ws.dk_part);
  a.dv_part = reinterpret_cast<float*>(base + ws.dv_part);
  a.pre_blocks = ws.pre_blocks;
  a.splits = ws.splits;
  const int fp32 = shape->dtype == ATTN_SINK_FP32;

  // The dQ kernel also writes the row statistics and the dS_h partials, so it runs
  // even without query rows (its workgroups then only write zero partials).
  st = timed_launch(K_BWD_DQ, stream, [&] { return launch_bwd_dq(a, fp32, stream); });
  if (st != ATTN_SINK_OK) return st;
  if (any_k) {
    st = timed_launch(K_BWD_DKDV, stream, [&] { return launch_bwd_dkdv(a, fp32, stream); });
    if (st != ATTN_SINK_OK) return st;
  }
  return timed_launch(K_BWD_FINISH, stream, [&] { return launch_bwd_finish(a, fp32, stream); });
}

attn_sink_status attn_sink_merge(int dtype, int head_dim, int num_heads_q, int total_q, int num_parts,
                                 const void* o_parts, const float* lse_parts, const float* sinks, void* o,
                                 float* lse, hipStream_t stream) {
  if (dtype != ATTN_SINK_BF16 && dtype != ATTN_SINK_FP32) return ATTN_SINK_ERR_UNSUPPORTED;
  if (!head_dim_built(head_dim)) return head_dim > 0 ? ATTN_SINK_ERR_UNSUPPORTED : ATTN_SINK_ERR_INVALID_ARG;
  if (num_heads_q < 1 || total_q < 0 || num_parts < 1) return ATTN_SINK_ERR_INVALID_ARG;
  if (!sinks) return ATTN_SINK_ERR_INVALID_ARG;
  if (total_q > 0 && (!o_parts || !lse_parts || !o || !lse)) return ATTN_SINK_ERR_INVALID_ARG;
  if (misaligned({o_parts, o}, {lse_parts, sinks, lse})) return ATTN_SINK_ERR_INVALID_ARG;
  if (total_q == 0) return ATTN_SINK_OK;
  MergeArgs a;
  a.o_parts = o_parts;
  a.lse_parts = lse_parts;
  a.sinks = sinks;
  a.o = o;
  a.lse = lse;
  a.parts = num_parts;
  a.hq = num_heads_q;
  a.total_q = total_q;
  a.d = head_dim;
  const int fp32 = dtype == ATTN_SINK_FP32;
  return timed_launch(K_MERGE, stream, [&] { return launch_merge(a, fp32, stream); });
}

const char* attn_sink_status_string(attn_sink_status status) {
  switch (status) {
    case ATTN_SINK_OK: return "ok";
    case ATTN_SINK_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_SINK_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_SINK_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case ATTN_SINK_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

attn_sink_status attn_sink_timing_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (enable) clear_records_locked();
  g_timing.store(enable != 0, std::memory_order_release);
  return ATTN_SINK_OK;
}

int attn_sink_timing_read(const char** names, int* launches, double* total_ms, int max) {
  std::lock_guard<std::mutex> lk(g_mu);
  int cnt[K_COUNT] = {0};
  double ms[K_COUNT] = {0};
  for (auto& r : g_records) {
    if (hipEventSynchronize(r.stop) != hipSuccess) return -1;
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess) return -1;
    cnt[r.kernel] += 1;
    ms[r.kernel] += t;
  }
  int n = 0;
  for (int k = 0; k < K_COUNT; ++k) {
    if (cnt[k] == 0) continue;
    if (n < max) {
      if (names) names[n] = kernel_name(k);
      if (launches) launches[n] = cnt[k];
      if (total_ms) total_ms[n] = ms[k];
    }
    ++n;
  }
  return n;
}

}  // extern "C"
