// Host-side layout of the backward and decoding workspaces, and the launch-shape
// choices they depend on (dQ row tiles, dK/dV head splits, decoding chunks).  Host
// code only: the C ABI carves the caller's workspace with these offsets and the
// launchers size their grids from the same functions.
#include "kernels.h"

namespace attn_sink {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Head-packed dQ tiles (as the forward's) on sliding-window layers: G = Hq / Hkv > 1
// dividing the 128 rows of a tile, and the (sequence x tile) grid row within 65535.
bool dq_head_packed(int hq, int hkv, int num_seqs, int max_q, int window) {
  constexpr int BM = kDqRows;
  const int G = hq / hkv;
  if (window <= 0 || G < 2 || BM % G != 0) return false;
  return ((long long)max_q * G + BM - 1) / BM * num_seqs <= 65535;
}

// Row tiles per sequence of the dQ grid (one dS_h partial per head and row tile).
int dq_tiles(int hq, int hkv, int num_seqs, int max_q, int window) {
  constexpr int BM = kDqRows;
  const int per = dq_head_packed(hq, hkv, num_seqs, max_q, window) ? BM / (hq / hkv) : BM;
  return (max_q + per - 1) / per;
}

int bwd_head_splits(int hq, int hkv, int total_k, int num_seqs, int causal, int window, int d, int fp32) {
  // The dK/dV grid has one workgroup per (sequence, kv head, head split, folded pair
  // of 128-key tiles); 256 or 512 run at once (one or two per compute unit, by the
  // variant's registers).  Splitting the
  // query heads of a kv head over s workgroups divides each workgroup's work by s
  // but multiplies the grid by s and adds float32 partials (written here, read back
  // by the finish kernel).  Estimated time, in microseconds:
  //   rounds(s) x (group / s) x steps x 2.25  +  partial bytes(s) / 5 TB/s
  // where steps is the number of (query head, 64-row tile) steps one folded pair
  // takes for one head (from the mean sequence length, the mask and the window) and
  // 2.25 us is the measured time of one such step.  Pick the cheapest s (the fewest
  // splits on a tie).
  const int group = hq / hkv;
  const long long bnb = kDkvKeys;  // keys per tile
  long long pairs = (total_k + 2 * bnb - 1) / (2 * bnb) + num_seqs / 2;  // folded pairs (approx.)
  if (pairs < 1) pairs = 1;
  const long long n = num_seqs > 0 ? (long long)total_k / num_seqs : total_k;  // mean sequence length
  long long steps;
  if (window > 0) {
    const long long w = window < n ? window : n;
    steps = 2 * ((w + bnb + 63) / 64 + 1);  // each tile of the pair sees about window + bnb rows
  } else {
    steps = causal ? n / 64 + bnb / 64 : 2 * (n / 64 + 1);
  }
  if (steps < 1) steps = 1;
  const long long kConcurrent = 256LL * ((!fp32 && d == 64) ? 2 : 1);  // resident dK/dV workgroups per compute unit: 2 (bf16, d = 64) or 1
  const double part_bytes = 2.0 * 2.0 * (double)total_k * hkv * d * 4.0;  // dK + dV, written and read, per split
  int best = 1;
  double best_t = 0.0;
  for (int sp = 1; sp <= group && group % sp == 0; sp *= 2) {
    const long long rounds = (pairs * hkv * sp + kConcurrent - 1) / kConcurrent;
    const double t = (double)rounds * (double)(group / sp) * (double)steps * 2.25 + (sp > 1 ? sp * part_bytes / 5e6 : 0.0);
    if (sp == 1 || t < best_t) {
      best = sp;
      best_t = t;
    }
  }
  return best;
}

BwdWorkspace bwd_workspace_layout(int hq, int hkv, int total_q, int total_k, int num_seqs, int max_q, int causal,
                                  int window, int d, int fp32) {
  BwdWorkspace w;
  // one dS_h partial per (head, sequence, dQ row tile): the dQ workgroups write them
  w.pre_blocks = num_seqs * dq_tiles(hq, hkv, num_seqs, max_q, window);
  w.splits = bwd_head_splits(hq, hkv, total_k, num_seqs, causal, window, d, fp32);
  size_t o = 0;
  w.rowstat = o;     o = align256(o + (size_t)hq * 2 * total_q * 4);
  w.dsink_part = o;  o = align256(o + (size_t)hq * w.pre_blocks * 4);
  const size_t part = w.splits > 1 ? (size_t)w.splits * total_k * hkv * d * 4 : 0;
  w.dk_part = o;     o = align256(o + part);
  w.dv_part = o;     o = align256(o + part);
  w.total = o;
  return w;
}

bool decode_supported(int hq, int hkv, int max_q) { return (long long)(hq / hkv) * max_q <= kDecodeCols; }

DecodeWorkspace decode_workspace_layout(int fp32, int hq, int hkv, int num_seqs, int max_q, int max_k, int window,
                                        int d) {
  DecodeWorkspace w;
  (void)fp32;
  // kv heads per workgroup: the largest divisor of hkv up to kDecodeWaves.
  w.hw = 1;
  for (int d = 1; d <= kDecodeWaves; ++d)
    if (hkv % d == 0) w.hw = d;
  // Visible key tiles of one sequence at most (a window may straddle one more tile).
  long long span = max_k;
  if (window > 0 && (long long)window + max_q - 1 < span) span = (long long)window + max_q - 1;
  const long long tiles = max_q > 0 ? (span + kDecodeKeys - 1) / kDecodeKeys + (window > 0 ? 1 : 0) : 0;
  // A fixed chunk, so a sequence's result depends on that sequence alone and not on
  // the rest of the batch (batch invariance: the same rounding order whatever the
  // batch size or the longest cache).  1024 keys: a partial costs under 1% of the
  // bytes its chunk reads, a 128-key window (at most 5 tiles) needs no merge, and a
  // 64-sequence rollout step of 1k-16k caches gives about a thousand workgroups.
  // The grid limit (65535 chunks) is far beyond max_seqlen_k <= 65535 * 128.
  const long long chunk = kDecodeChunk;
  (void)num_seqs;
  w.chunk = (int)chunk;
  w.max_chunks = (int)(tiles > 0 ? (tiles + chunk - 1) / chunk : 1);
  w.cols = (hq / hkv) * max_q;
  if (w.cols < 1) w.cols = 1;
  const size_t parts = w.max_chunks > 1 ? (size_t)num_seqs * hkv * w.max_chunks * w.cols : 0;
  w.part_o = 0;
  w.part_ml = (parts * d * sizeof(float) + 255) & ~(size_t)255;
  w.total = w.part_ml + ((parts * 2 * sizeof(float) + 255) & ~(size_t)255);
  if (w.total == 0) w.total = 256;  // nothing to keep, but a valid shape never reports 0
  return w;
}

}  // namespace attn_sink
