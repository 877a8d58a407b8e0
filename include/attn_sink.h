/*
 * attn_sink.h - C ABI of the MI355X (gfx950) attention-with-learnable-sinks library.
 *
 * What is computed.  For every sequence b of a packed batch and every query
 * head h (kv head g = h / (Hq / Hkv)):
 *
 *   s_ij     = softmax_scale * <q_i, k_j>                     for visible keys j
 *   P_ij     = exp(s_ij) / (sum_j' exp(s_ij') + exp(S_h))
 *   P_sink_i = exp(S_h)  / (same denominator)
 *   o_i      = sum_j P_ij v_j                  (the sink is never multiplied by V)
 *   lse_i    = log(sum_j exp(s_ij) + exp(S_h))  (natural log, the sink included)
 *
 * This is the sink softmax of "Unlocking Agentic RL Training for GPT-OSS"
 * (euno.news, zh), section on attention-sink support in FlashAttention V3:
 * sub-section 带汇聚的注意力 (one learnable logit S_h per head appended to every
 * score row as a virtual key, dropped before the product with V) and
 * sub-section 数学公式 (the two probability formulas above).  The backward
 * returns dq, dk, dv and the sink gradient of sub-section 反向传播,
 * dS_h = -sum_i P_sink_i * D_i with D_i = <dO_i, o_i>.
 *
 * Visibility (masks are not on the pages; this ABI defines them): key j of a
 * sequence with n_q queries and n_k keys is visible to query i when
 *   (causal == 0 || j <= i + n_k - n_q) && (window <= 0 || j > i + n_k - n_q - window).
 * "window = W" therefore means W keys including the diagonal.  The sink is
 * visible to every row.
 *
 * Layouts (all contiguous, row-major, element type given by dtype):
 *   q, o, dout, dq : [total_q, Hq,  head_dim]
 *   k, v, dk, dv   : [total_k, Hkv, head_dim]
 *   lse            : [Hq, total_q] float32, natural log, includes the sink
 *   sinks, dsinks  : [Hq] float32, in score units (not multiplied by softmax_scale)
 *   cu_seqlens_q/k : [num_seqs + 1] int32, DEVICE memory, cu[0] = 0, nondecreasing,
 *                    cu[num_seqs] = total.  Fixed-length batches use [0, N, 2N, ...].
 * Alignment: the kernels move q, k, v, o, dout, dq, dk, dv (and the merge's o_parts)
 * in 16-byte pieces, so these pointers must be 16-byte aligned; the float32 and
 * int32 arrays need their natural 4 bytes.  A misaligned pointer is
 * ATTN_SINK_ERR_INVALID_ARG.  Whole allocations and row slices of contiguous
 * tensors always qualify.
 *
 * Ownership: the caller allocates every buffer (device memory for all tensors,
 * including the backward workspace).  The library allocates no device memory,
 * keeps no state between calls (apart from the opt-in timing records below),
 * never synchronises the stream, and enqueues all work on `stream` in order.
 * Outputs (o, lse, dq, dk, dv, dsinks) are overwritten, not accumulated.
 *
 * Errors: every argument check runs on the host before anything is enqueued, so
 * a status of ATTN_SINK_ERR_INVALID_ARG, _UNSUPPORTED or _WORKSPACE means nothing
 * has been enqueued.  ATTN_SINK_ERR_HIP reports a launch error taken from the HIP
 * runtime; an entry point that launches several kernels (attn_sink_bwd,
 * attn_sink_fwd_decode) may by then have enqueued the kernels before the one that
 * failed, and its outputs are then undefined.  Faults inside a kernel are
 * asynchronous and surface at the caller's next synchronisation.  The kernels
 * clamp cu_seqlens entries to [0, total] before use, so a malformed cu_seqlens
 * gives wrong numbers but no out-of-bounds access; sequences longer than
 * max_seqlen_* are only partly computed (caller contract: max_seqlen_* >= every
 * sequence length).
 *
 * Thread safety: calls are reentrant; concurrent calls on different streams are
 * independent (they must not share output or workspace buffers).
 *
 * Graph capture: no entry point allocates, sets memory or synchronises, so every
 * call can be captured into a HIP graph on `stream` (with the timing records off);
 * each replay overwrites every output, so it depends on its inputs alone.
 */
#ifndef ATTN_SINK_H
#define ATTN_SINK_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_SINK_OK = 0,
  ATTN_SINK_ERR_INVALID_ARG = 1,  /* null or misaligned pointer, bad count, Hq % Hkv != 0, ... */
  ATTN_SINK_ERR_UNSUPPORTED = 2,  /* well-formed but not built: head_dim not 64 or 128, dtype, decode width */
  ATTN_SINK_ERR_WORKSPACE = 3,    /* workspace missing, misaligned or smaller than required */
  ATTN_SINK_ERR_HIP = 4           /* the HIP runtime refused a launch */
} attn_sink_status;

typedef enum {
  ATTN_SINK_BF16 = 0,  /* q, k, v, o, dout, dq, dk, dv in bfloat16; MFMA bf16 x bf16 -> fp32 */
  ATTN_SINK_FP32 = 1   /* the same tensors in float32; MFMA fp32 x fp32 -> fp32 */
} attn_sink_dtype;

typedef struct {
  int dtype;               /* attn_sink_dtype */
  int head_dim;            /* 64 or 128 */
  int num_heads_q;         /* Hq  >= 1 */
  int num_heads_kv;        /* Hkv >= 1, Hq % Hkv == 0 (GQA: heads h of one kv head are contiguous) */
  int num_seqs;            /* >= 1 */
  int total_q;             /* rows of q / o (>= 0) */
  int total_k;             /* rows of k / v (>= 0) */
  int max_seqlen_q;        /* >= every query length; sizes the launch grid */
  int max_seqlen_k;        /* >= every key length */
  const int* cu_seqlens_q; /* device, [num_seqs + 1] */
  const int* cu_seqlens_k; /* device, [num_seqs + 1] */
  float softmax_scale;     /* multiplies q.k (e.g. 1/sqrt(head_dim)); finite, > 0 */
  int causal;              /* 0 or 1 */
  int window;              /* <= 0: none; else W keys including the diagonal */
} attn_sink_shape;

/* Forward (sub-sections 带汇聚的注意力 and 数学公式 of the page cited above).
 * Writes o (dtype) and lse (float32).  sinks may hold -INFINITY (then the head
 * is standard attention); a row that sees no key and has S_h = -inf gets
 * o = 0 and lse = -inf.  +INFINITY sinks are outside the domain. */
attn_sink_status attn_sink_fwd(const attn_sink_shape* shape,
                               const void* q, const void* k, const void* v,
                               const float* sinks,
                               void* o, float* lse,
                               hipStream_t stream);

/* Forward for a few new query rows per sequence against long key ranges: a
 * decoding step, or a short chunk, against a KV cache.  Same function, inputs,
 * layouts, masks and outputs as attn_sink_fwd (sub-sections 带汇聚的注意力 and
 * 数学公式 of the page cited above), organised for this shape: the key range of
 * every (sequence, kv head) is split over many workgroups that each keep an
 * online softmax without the sink, and a merge kernel combines the splits in a
 * fixed order and adds exp(S_h) to the normaliser exactly once.  The results equal
 * attn_sink_fwd's up to floating-point rounding order (not bitwise) and are
 * bitwise reproducible from run to run.
 * Requires (Hq / Hkv) * max_seqlen_q <= 32 (the query heads of one kv head times
 * the new rows of one sequence share one 32-column matrix-core block), else
 * ATTN_SINK_ERR_UNSUPPORTED; rows are bottom-right aligned with the keys, as in
 * attn_sink_fwd (row i of n_q sits at key position i + n_k - n_q).
 * workspace: device memory of at least attn_sink_fwd_decode_workspace_bytes(shape)
 * bytes, 256-byte aligned, owned by the caller, contents need not be initialised
 * and are garbage afterwards; ATTN_SINK_ERR_WORKSPACE if missing, misaligned or
 * too small. */
attn_sink_status attn_sink_fwd_decode(const attn_sink_shape* shape,
                                      const void* q, const void* k, const void* v,
                                      const float* sinks,
                                      void* o, float* lse,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* Bytes of device workspace attn_sink_fwd_decode needs for `shape` (0 on an
 * invalid or unsupported shape). */
size_t attn_sink_fwd_decode_workspace_bytes(const attn_sink_shape* shape);

/* Bytes of the fixed scratch attn_sink_fwd_decode_noalloc works in. */
#define ATTN_SINK_DECODE_SCRATCH_BYTES ((size_t)64 << 20)

/* attn_sink_fwd_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments (minus the workspace), the
 * same kernels and bitwise the same results.  The partials live in a fixed
 * scratch array of ATTN_SINK_DECODE_SCRATCH_BYTES that the library holds on each
 * GPU it runs on, from that device's first call until the process ends; the call
 * itself allocates nothing (no hipMalloc, no events: it records no timing).
 * The scratch used is the current device's: `stream` must belong to the current
 * device (else ATTN_SINK_ERR_INVALID_ARG).  A shape whose workspace
 * (attn_sink_fwd_decode_workspace_bytes) exceeds ATTN_SINK_DECODE_SCRATCH_BYTES
 * returns ATTN_SINK_ERR_WORKSPACE before anything is enqueued.  Every call on one
 * GPU shares that GPU's scratch and finds the previous call's contents there (no
 * part of it needs clearing: every partial read is written first by the same
 * call); calls that overlap in time on one GPU (different streams or threads) race
 * on it and must be serialised by the caller. */
attn_sink_status attn_sink_fwd_decode_noalloc(const attn_sink_shape* shape,
                                              const void* q, const void* k, const void* v,
                                              const float* sinks,
                                              void* o, float* lse,
                                              hipStream_t stream);

/* Bytes of device workspace attn_sink_bwd needs for `shape` (0 on invalid shape). */
size_t attn_sink_bwd_workspace_bytes(const attn_sink_shape* shape);

/* Backward of attn_sink_fwd for upstream gradient dout (sub-section 反向传播 of
 * the page cited above for dsinks; dq, dk, dv by the chain rule through the
 * softmax over the score row with the sink column appended).
 * o and lse must be the forward's outputs for the same inputs.  Writes dq (dtype,
 * layout of q), dk/dv (dtype, layout of k) and dsinks (float32, [Hq]).
 * dsinks_h = -sum_i P_sink_i D_i is formed with D_i = sum_j P_ij dP_ij from the
 * float32 probabilities the call recomputes, as
 *   -sum_i P_sink_i (sum_j dS_ij + D'_i (1 - P_sink_i)),  D'_i = <dout_i, o_i>,
 * which is exact when the call sees every key of each row (sum_j P_ij =
 * 1 - P_sink_i).  D'_i alone would carry the rounding of o into a sum whose terms
 * can cancel to a small fraction of their size.  A call over a shard of the keys
 * returns its shard's part plus the key-free term -sum_i P_sink_i D'_i
 * (1 - P_sink_i) (see attn_sink_merge for combining shards).
 * workspace: device memory of at least attn_sink_bwd_workspace_bytes(shape)
 * bytes, 256-byte aligned, owned by the caller, contents need not be initialised
 * and are garbage afterwards.  No atomics are used: dq is produced by one
 * workgroup per query block, dk/dv by one per key block (summing the query heads
 * of a kv head in a fixed order, through float32 partials in the workspace when
 * the heads are split across workgroups), and dsinks by a fixed-order reduction,
 * so every output is bitwise reproducible from run to run. */
attn_sink_status attn_sink_bwd(const attn_sink_shape* shape,
                               const void* q, const void* k, const void* v,
                               const float* sinks,
                               const void* o, const float* lse, const void* dout,
                               void* dq, void* dk, void* dv, float* dsinks,
                               void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Merge of attention partials over disjoint key shards into sink attention, the
 * sink counted exactly once.  This is the combine step of sequence (context)
 * parallelism, where each device attends its query rows to one shard of the keys at
 * a time (sequence parallelism for long rollouts: keryc.com "GPT-OSS enables agentic
 * RL training", section Solutions; the normaliser with one exp(S_h): "Unlocking
 * Agentic RL Training for GPT-OSS", 数学公式).
 * Part s is what attn_sink_fwd returns for the same query rows against shard s's
 * keys with every sink set to -INFINITY: o_parts[s] the standard-attention output
 * over the shard, lse_parts[s] its natural-log normaliser (-inf where a row sees no
 * key of the shard).  Writes, with the sinks given here,
 *   M = max(S_h, max_s lse_s),  L = exp(S_h - M) + sum_s exp(lse_s - M),
 *   o = sum_s exp(lse_s - M) o_s / L,  lse = M + log L,
 * which equal attn_sink_fwd over all the keys up to rounding.  Parts are folded in
 * index order (bitwise repeatable).
 * Layouts: o_parts [num_parts, total_q, Hq, head_dim] (dtype), lse_parts
 * [num_parts, Hq, total_q] float32, sinks [Hq] float32, o [total_q, Hq, head_dim]
 * (dtype), lse [Hq, total_q] float32.  Outputs must not alias the inputs.
 * The backward of the sharded attention needs no merge kernel: calling
 * attn_sink_bwd per shard with the merged o and lse gives that shard's dk, dv and
 * its share of dq (summed over the shards).  Each such call's dsinks is its
 * shard's part of the sink gradient plus a term that does not depend on the keys
 * (see attn_sink_bwd), which a call with no keys (total_k = 0) returns alone:
 * over n shards, dsinks = sum of the shard calls' dsinks - (n - 1) x that call's.
 * Errors: ATTN_SINK_ERR_UNSUPPORTED for dtype / head_dim; ATTN_SINK_ERR_INVALID_ARG
 * for num_heads_q < 1, total_q < 0, num_parts < 1 or a null pointer. */
attn_sink_status attn_sink_merge(int dtype, int head_dim, int num_heads_q, int total_q, int num_parts,
                                 const void* o_parts, const float* lse_parts,
                                 const float* sinks,
                                 void* o, float* lse,
                                 hipStream_t stream);

/* Static, human-readable name of a status code. */
const char* attn_sink_status_string(attn_sink_status status);

/* Opt-in per-kernel timing for measurement harnesses.  While enabled, every
 * kernel the compute entry points launch is bracketed by HIP events on the launch
 * stream (this adds event records to the stream, nothing else).
 * attn_sink_timing_enable(1) clears earlier records; (0) stops recording.
 * attn_sink_timing_read synchronises on the recorded events and fills, for up to
 * `max` kernels, the kernel name, the number of launches and the summed duration
 * in milliseconds; it returns the number of distinct kernels (or -1 on error).
 * Names point to static strings.  Not thread-safe: one harness at a time. */
attn_sink_status attn_sink_timing_enable(int enable);
int attn_sink_timing_read(const char** names, int* launches, double* total_ms, int max);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_SINK_H */
