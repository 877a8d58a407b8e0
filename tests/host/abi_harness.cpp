// Host-only harness for the C ABI layer (api.cpp) and the workspace layout
// (layout.cpp), built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py.  The HIP runtime calls and the kernel launchers
// are replaced by stubs: each launcher stub writes every byte of every workspace
// region the kernels would write (so a carve-up that overlaps or overruns the
// caller's workspace, which is allocated here at exactly the reported size, is a
// heap overflow the sanitizer reports), and the event stubs count live events
// (so a record leaked on an error path shows up, also to LeakSanitizer).
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "attn_sink.h"
#include "kernels.h"

// ---------------------------------------------------------------- HIP runtime stubs
static int g_live_events = 0;
static int g_record_calls = 0;
static int g_fail_record_at = -1;  // the n-th hipEventRecord call fails (-1: never)
static int g_current_device = 0;

extern "C" {
hipError_t hipEventCreate(hipEvent_t* e) {
  *e = reinterpret_cast<hipEvent_t>(new int(7));
  ++g_live_events;
  return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t e) {
  delete reinterpret_cast<int*>(e);
  --g_live_events;
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) {
  return g_record_calls++ == g_fail_record_at ? hipErrorInvalidValue : hipSuccess;
}
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
  *ms = 1.0f;
  return hipSuccess;
}
hipError_t hipGetDevice(int* d) {
  *d = g_current_device;
  return hipSuccess;
}
// Fake streams carry their device in the pointer value: (device + 1) * 0x1000.
hipError_t hipStreamGetDevice(hipStream_t s, hipDevice_t* d) {
  *d = (int)(reinterpret_cast<uintptr_t>(s) / 0x1000) - 1;
  return hipSuccess;
}
}

// ---------------------------------------------------------------- launcher stubs
namespace attn_sink {
static int g_launches = 0;
static bool g_fail_launch = false;
static std::vector<unsigned char> g_scratch(kDecodeScratchBytes);

static hipError_t done() {
  ++g_launches;
  return g_fail_launch ? hipErrorLaunchFailure : hipSuccess;
}
static void touch(void* p, size_t bytes) {
  if (bytes) std::memset(p, 0x5a, bytes);
}

hipError_t launch_fwd(const FwdArgs&, int, hipStream_t) { return done(); }
hipError_t launch_merge(const MergeArgs&, int, hipStream_t) { return done(); }
hipError_t launch_bwd_dq(const BwdArgs& a, int, hipStream_t) {
  touch(a.rowstat, (size_t)a.f.hq * 2 * a.f.total_q * 4);
  touch(a.dsink_part, (size_t)a.f.hq * a.pre_blocks * 4);
  return done();
}
hipError_t launch_bwd_dkdv(const BwdArgs& a, int, hipStream_t) {
  if (a.splits > 1) {
    const size_t part = (size_t)a.splits * a.f.total_k * a.f.hkv * a.f.d * 4;
    touch(a.dk_part, part);
    touch(a.dv_part, part);
  }
  return done();
}
hipError_t launch_bwd_finish(const BwdArgs&, int, hipStream_t) { return done(); }
hipError_t launch_decode_partial(const DecodeArgs& a, int, hipStream_t) {
  if (a.max_chunks > 1) {
    const size_t slots = (size_t)a.f.num_seqs * a.f.hkv * a.max_chunks * a.cols;
    touch(a.part_o, slots * a.f.d * 4);
    touch(a.part_ml, slots * 2 * 4);
  }
  return done();
}
hipError_t launch_decode_merge(const DecodeArgs&, int, hipStream_t) { return done(); }
hipError_t decode_scratch(void** p) {
  *p = g_scratch.data();
  return hipSuccess;
}
}  // namespace attn_sink

// ---------------------------------------------------------------- checks
static int g_checks = 0, g_failures = 0;
#define CHECK(cond)                                                  \
  do {                                                               \
    ++g_checks;                                                      \
    if (!(cond)) {                                                   \
      ++g_failures;                                                  \
      std::printf("FAILED line %d: %s\n", __LINE__, #cond);         \
    }                                                                \
  } while (0)

static const void* const FAKE = reinterpret_cast<const void*>(0x100000);  // never dereferenced
static int g_cu[2] = {0, 0};

static attn_sink_shape shape(int dtype, int d, int hq, int hkv, int seqs, int tq, int tk, int mq, int mk,
                             int causal, int window) {
  attn_sink_shape s;
  s.dtype = dtype;
  s.head_dim = d;
  s.num_heads_q = hq;
  s.num_heads_kv = hkv;
  s.num_seqs = seqs;
  s.total_q = tq;
  s.total_k = tk;
  s.max_seqlen_q = mq;
  s.max_seqlen_k = mk;
  s.cu_seqlens_q = g_cu;
  s.cu_seqlens_k = g_cu;
  s.softmax_scale = 0.125f;
  s.causal = causal;
  s.window = window;
  return s;
}

static void* alloc256(size_t bytes) {
  void* p = nullptr;
  if (posix_memalign(&p, 256, bytes ? bytes : 1) != 0) std::abort();
  return p;
}

static void backward_case(const attn_sink_shape& s) {
  const size_t need = attn_sink_bwd_workspace_bytes(&s);
  CHECK(need > 0);
  void* ws = alloc256(need);  // exactly the reported size: an overrun is a heap overflow
  float dsinks[128];
  const void* f = FAKE;
  CHECK(attn_sink_bwd(&s, f, f, f, (const float*)f, f, (const float*)f, f, (void*)f, (void*)f, (void*)f, dsinks, ws,
                      need - 1, nullptr) == ATTN_SINK_ERR_WORKSPACE);
  CHECK(attn_sink_bwd(&s, f, f, f, (const float*)f, f, (const float*)f, f, (void*)f, (void*)f, (void*)f, dsinks,
                      (char*)ws + 16, need, nullptr) == ATTN_SINK_ERR_WORKSPACE);  // misaligned
  CHECK(attn_sink_bwd(&s, f, f, f, (const float*)f, f, (const float*)f, f, (void*)f, (void*)f, (void*)f, dsinks, ws,
                      need, nullptr) == ATTN_SINK_OK);
  std::free(ws);
}

static void decode_case(const attn_sink_shape& s) {
  const size_t need = attn_sink_fwd_decode_workspace_bytes(&s);
  CHECK(need > 0);
  void* ws = alloc256(need);
  const void* f = FAKE;
  CHECK(attn_sink_fwd_decode(&s, f, f, f, (const float*)f, (void*)f, (float*)f, ws, need, nullptr) == ATTN_SINK_OK);
  std::free(ws);
  const bool fits = need <= ATTN_SINK_DECODE_SCRATCH_BYTES;
  CHECK(attn_sink_fwd_decode_noalloc(&s, f, f, f, (const float*)f, (void*)f, (float*)f, nullptr) ==
        (fits ? ATTN_SINK_OK : ATTN_SINK_ERR_WORKSPACE));
}

int main() {
  const void* f = FAKE;
  // Argument checks: nothing is launched.
  attn_sink_shape s = shape(ATTN_SINK_BF16, 64, 64, 8, 1, 4096, 4096, 4096, 4096, 1, 0);
  CHECK(attn_sink_fwd(nullptr, f, f, f, (const float*)f, (void*)f, (float*)f, nullptr) == ATTN_SINK_ERR_INVALID_ARG);
  attn_sink_shape bad = s;
  bad.head_dim = 96;
  CHECK(attn_sink_fwd(&bad, f, f, f, (const float*)f, (void*)f, (float*)f, nullptr) == ATTN_SINK_ERR_UNSUPPORTED);
  bad = s;
  bad.num_heads_q = 63;
  CHECK(attn_sink_fwd(&bad, f, f, f, (const float*)f, (void*)f, (float*)f, nullptr) == ATTN_SINK_ERR_INVALID_ARG);
  CHECK(attn_sink_fwd(&s, (const char*)f + 8, f, f, (const float*)f, (void*)f, (float*)f, nullptr) ==
        ATTN_SINK_ERR_INVALID_ARG);  // misaligned q
  CHECK(attn_sink_bwd_workspace_bytes(&bad) == 0);
  CHECK(attn_sink_merge(ATTN_SINK_BF16, 64, 8, 10, 0, f, (const float*)f, (const float*)f, (void*)f, (float*)f,
                        nullptr) == ATTN_SINK_ERR_INVALID_ARG);
  CHECK(attn_sink_status_string((attn_sink_status)99) != nullptr);
  CHECK(attn_sink::g_launches == 0);

  // Backward workspaces: causal 4k (head splits), window layers (head-packed dS_h
  // partials), several sequences, head dim 128, fp32, one kv head, no keys.
  backward_case(s);
  backward_case(shape(ATTN_SINK_BF16, 64, 64, 8, 1, 16384, 16384, 16384, 16384, 1, 128));
  backward_case(shape(ATTN_SINK_BF16, 64, 64, 8, 8, 49802, 49802, 14090, 14090, 1, 0));
  backward_case(shape(ATTN_SINK_BF16, 64, 64, 8, 8, 49802, 49802, 14090, 14090, 1, 128));
  backward_case(shape(ATTN_SINK_BF16, 128, 32, 8, 1, 4096, 4096, 4096, 4096, 1, 0));
  backward_case(shape(ATTN_SINK_FP32, 64, 2, 1, 1, 64, 64, 64, 64, 1, 0));
  backward_case(shape(ATTN_SINK_BF16, 64, 16, 1, 3, 900, 900, 300, 300, 0, 0));
  backward_case(shape(ATTN_SINK_BF16, 64, 8, 2, 3, 900, 0, 300, 0, 0, 0));

  // Decoding workspaces: one new row, several rows, a window, head dim 128; the
  // allocation-free call on the same shapes, and one beyond its scratch.
  decode_case(shape(ATTN_SINK_BF16, 64, 64, 8, 64, 64, 542080, 1, 16372, 1, 0));
  decode_case(shape(ATTN_SINK_BF16, 64, 64, 8, 64, 64, 542080, 1, 16372, 1, 128));
  decode_case(shape(ATTN_SINK_BF16, 64, 16, 4, 5, 20, 50000, 4, 20000, 1, 0));
  decode_case(shape(ATTN_SINK_BF16, 128, 32, 8, 4, 16, 40000, 4, 10000, 1, 0));
  decode_case(shape(ATTN_SINK_BF16, 64, 64, 8, 64, 256, 64 * 65535, 4, 65535, 1, 0));

  // The allocation-free call on a stream of another device is refused.
  attn_sink_shape d1 = shape(ATTN_SINK_BF16, 64, 64, 8, 4, 4, 4000, 1, 1000, 1, 0);
  hipStream_t dev1 = reinterpret_cast<hipStream_t>(2 * 0x1000);  // device 1
  hipStream_t dev0 = reinterpret_cast<hipStream_t>(1 * 0x1000);  // device 0
  CHECK(attn_sink_fwd_decode_noalloc(&d1, f, f, f, (const float*)f, (void*)f, (float*)f, dev1) ==
        ATTN_SINK_ERR_INVALID_ARG);
  CHECK(attn_sink_fwd_decode_noalloc(&d1, f, f, f, (const float*)f, (void*)f, (float*)f, dev0) == ATTN_SINK_OK);

  // Timing records: every launch adds one record (two events); a failed event
  // record or launch releases its events.
  CHECK(attn_sink_timing_enable(1) == ATTN_SINK_OK);
  CHECK(attn_sink_fwd(&s, f, f, f, (const float*)f, (void*)f, (float*)f, nullptr) == ATTN_SINK_OK);
  CHECK(g_live_events == 2);
  g_fail_record_at = g_record_calls + 1;  // the stop event of the next launch
  CHECK(attn_sink_fwd(&s, f, f, f, (const float*)f, (void*)f, (float*)f, nullptr) == ATTN_SINK_ERR_HIP);
  CHECK(g_live_events == 2);
  g_fail_record_at = g_record_calls;  // the start event of the next launch
  CHECK(attn_sink_fwd(&s, f, f, f, (const float*)f, (void*)f, (float*)f, nullptr) == ATTN_SINK_ERR_HIP);
  CHECK(g_live_events == 2);
  g_fail_record_at = -1;
  attn_sink::g_fail_launch = true;
  CHECK(attn_sink_fwd(&s, f, f, f, (const float*)f, (void*)f, (float*)f, nullptr) == ATTN_SINK_ERR_HIP);
  CHECK(g_live_events == 2);
  attn_sink::g_fail_launch = false;
  const char* names[8];
  int launches[8];
  double ms[8];
  CHECK(attn_sink_timing_read(names, launches, ms, 8) == 1);
  CHECK(launches[0] == 1 && ms[0] == 1.0 && std::strcmp(names[0], "attn_sink_fwd_kernel") == 0);
  CHECK(attn_sink_timing_enable(1) == ATTN_SINK_OK);  // clears the records
  CHECK(g_live_events == 0);
  CHECK(attn_sink_timing_enable(0) == ATTN_SINK_OK);

  std::printf("abi harness: %d checks, %d failed, %d stub launches\n", g_checks, g_failures, attn_sink::g_launches);
  return g_failures == 0 ? 0 : 1;
}
