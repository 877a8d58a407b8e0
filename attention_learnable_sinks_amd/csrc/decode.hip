// Forward of attention with per-head learnable sinks for a few query rows per
// sequence against long key ranges (a decoding step, or a short chunk, against a KV
// cache), on gfx950.
//
// Same function as the forward kernel -- per query row i of head h
//   o_i = sum_j P_ij v_j,  P_ij = exp(s_ij) / (sum_j' exp(s_ij') + exp(S_h)),
//   lse_i = log(sum_j exp(s_ij) + exp(S_h))
// ("Unlocking Agentic RL Training for GPT-OSS", 带汇聚的注意力 and 数学公式: the sink
// joins the normaliser once and never multiplies V) -- organised for the inference
// side, where each sequence contributes one or a few new rows and the key range is
// long:
//   * The query heads that share a kv head, times the new rows, fill the 32 columns
//     of one MFMA block (column c = query head g*G + c % G, row c / G), so K and V
//     are read once per kv head instead of once per query head.
//   * The key range is split over many workgroups (split-K); each of a workgroup's
//     four wavefronts streams every fourth key tile through its own LDS region and
//     keeps an exact online softmax (running max per tile, no sink).  The wavefronts
//     combine in a fixed order into one partial (O unnormalised, max m, sum l).
//   * A merge kernel combines the partials of a row in split order and adds the
//     sink's mass exactly once there:
//       M = max(S_h, max_s m_s),  L = e^(S_h - M) + sum_s l_s e^(m_s - M),
//       o = sum_s O_s e^(m_s - M) / L,  lse = M + log L      (exp2 domain inside)
//   The results equal the forward kernel's up to rounding order; the summation
//   order is fixed, so they are bitwise repeatable.
#include "common.h"
#include "kernels.h"

namespace attn_sink {

constexpr int kDecBN = 64;       // keys per tile
constexpr int kDecCols = 32;     // (query head, row) columns per kv head
constexpr int kDecWaves = 4;     // wavefronts per workgroup

template <typename T>
__global__ __launch_bounds__(256) void decode_partial_kernel(DecodeArgs a) {
  using M = Mfma<T>;
  using Frag = typename M::Frag;
  constexpr int E = M::E, KS = M::KS;
  constexpr int NQ = kD / KS;      // operand steps over the head dim
  constexpr int NP = kDecBN / KS;  // operand steps over the keys of a tile
  constexpr int TILE = tile_elems<T>(kDecBN);
  // Per wavefront: one K and one V tile.  Reused for the cross-wavefront combine.
  __shared__ __attribute__((aligned(16))) T smem[kDecWaves * 2 * TILE];
  static_assert(sizeof(smem) >= kDecWaves * kDecCols * (kD + 3) * sizeof(float), "combine buffer");

  const FwdArgs& f = a.f;
  const int grp = blockIdx.x;  // sequence * hkv + kv head
  const int b = grp / f.hkv, g = grp % f.hkv;
  const int split = blockIdx.y;
  const int G = f.hq / f.hkv;
  const SeqBounds sq = seq_bounds(f.cu_q, b, f.total_q);
  const SeqBounds sk = seq_bounds(f.cu_k, b, f.total_k);
  const int nq = sq.len, nk = sk.len, off = nk - nq;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, c = lane & 31;

  // Column c of the block: query head g*G + c % G, row c / G (valid while < nq).
  const int col_row = c / G, col_head = g * G + c % G;
  const bool col_ok = c < G * (kDecCols / G) && col_row < nq;
  Span keys = keys_of_row(col_row, off, nk, f.causal, f.window);
  if (!col_ok) keys.len = 0u;

  // Key tiles the rows of this kv head see, and this split's share of them.
  const Span first = keys_of_row(0, off, nk, f.causal, f.window);
  const Span last = keys_of_row(max(nq - 1, 0), off, nk, f.causal, f.window);
  const int klo = nq > 0 ? first.lo : 0;
  const int khi = nq > 0 ? last.lo + (int)last.len : 0;
  const int tb = klo / kDecBN;
  const int te = khi > klo ? (khi + kDecBN - 1) / kDecBN : tb;
  const int per = (te - tb + a.splits - 1) / a.splits;
  const int t0 = min(tb + split * per, te), t1 = min(t0 + per, te);

  Frag qf[NQ];
  {
    const T* src = static_cast<const T*>(f.q) + ((size_t)(sq.start + (col_ok ? col_row : 0)) * f.hq +
                                                 (col_ok ? col_head : 0)) * kD;
#pragma unroll
    for (int s = 0; s < NQ; ++s) qf[s] = global_frag<T>(src + KS * s + E * h, col_ok);
  }
  const float sl2 = f.scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;

  const size_t kv_row = (size_t)f.hkv * kD;
  T* const Ks = smem + w * 2 * TILE;
  T* const Vs = Ks + TILE;
  FragAddr<T> fa;
  fa.init(lane);
  TileLoader<T, kDecBN, 64> kld, vld;  // one wavefront moves its own tiles
  kld.init(static_cast<const T*>(f.k) + (size_t)sk.start * kv_row + g * kD, kv_row, nk, lane);
  vld.init(static_cast<const T*>(f.v) + (size_t)sk.start * kv_row + g * kD, kv_row, nk, lane);
  vmem_drain();

  for (int t = t0 + w; t < t1; t += kDecWaves) {
    // The previous tile's LDS reads have all returned: their MFMAs were issued.
    kld.issue(t * kDecBN, Ks);
    vld.issue(t * kDecBN, Vs);
    kld.finish();
    vld.finish();
    // The tile is this wavefront's alone: its own wait suffices (no workgroup barrier).
    // As asm with a memory clobber it also keeps the compiler from moving the LDS
    // reads of the tile above it.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    f32x16 st[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[mt][r] = 0.f;
#pragma unroll
      for (int s = 0; s < NQ; ++s) st[mt] = M::mma(fa.row(Ks, mt, s), qf[s], st[mt]);
    }
    // Mask to the column's visible keys (key of register r: t*BN + 4h + 32mt + 8(r/4) + r%4).
    const int k0 = t * kDecBN + 4 * h;
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        st[mt][r] = in_span(k0 + 32 * mt + 8 * (r / 4) + r % 4, keys) ? st[mt][r] : -INFINITY;
        mx = fmaxf(mx, st[mt][r]);
      }
    const float m_new = fmaxf(m_run, halves_max(mx) * sl2);
    const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);  // 0 when m_run = -inf
    const float neg_m = m_new == -INFINITY ? 0.f : -m_new;
    l_run *= alpha;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[t2][r] *= alpha;
    m_run = m_new;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) st[mt][r] = fast_exp2(fmaf(st[mt][r], sl2, neg_m));
#pragma unroll
    for (int s = 0; s < NP; ++s) {
      const Frag pf = pack_frag<T>(st, s);
      l_run = frag_sum<T>(pf, l_run);  // the sum of the rounded P that multiplies V
#pragma unroll
      for (int md = 0; md < 2; ++md) oacc[md] = M::mma(fa.col(Vs, md, s), pf, oacc[md]);
    }
  }
  const float l_col = halves_sum(l_run);

  // ---- combine the four wavefronts (fixed order) into this split's partial.
  __syncthreads();  // every wavefront is done with its tiles
  constexpr int OS = kD + 1;  // padded row: the 32 columns of a store hit 32 banks
  float* const o_s = reinterpret_cast<float*>(smem);   // [wave][col][d]
  float* const m_s = o_s + kDecWaves * kDecCols * OS;  // [wave][col]
  float* const l_s = m_s + kDecWaves * kDecCols;       // [wave][col]
#pragma unroll
  for (int md = 0; md < 2; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) o_s[(w * kDecCols + c) * OS + 32 * md + crow(r, h)] = oacc[md][r];
  if (h == 0) {
    m_s[w * kDecCols + c] = m_run;
    l_s[w * kDecCols + c] = l_col;
  }
  __syncthreads();
  float* const po = a.part_o + ((size_t)grp * a.splits + split) * kDecCols * kD;
  float* const pml = a.part_ml + ((size_t)grp * a.splits + split) * kDecCols * 2;
  for (int i = tid; i < kDecCols * kD; i += blockDim.x) {
    const int cc = i / kD, d = i % kD;
    float mm = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) mm = fmaxf(mm, m_s[ww * kDecCols + cc]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) {
      const float mw = m_s[ww * kDecCols + cc];
      const float sc = mw == -INFINITY ? 0.f : fast_exp2(mw - mm);
      o += o_s[(ww * kDecCols + cc) * OS + d] * sc;
      l += l_s[ww * kDecCols + cc] * sc;
    }
    po[i] = o;
    if (d == 0) {
      pml[2 * cc] = mm;
      pml[2 * cc + 1] = l;
    }
  }
}


// One workgroup per (sequence, kv head, four columns); thread = (column, d).
template <typename T>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  const FwdArgs& f = a.f;
  const int grp = blockIdx.x;
  const int b = grp / f.hkv, g = grp % f.hkv;
  const int G = f.hq / f.hkv;
  const int cc = 4 * blockIdx.y + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), d = threadIdx.x & 63;
  const SeqBounds sq = seq_bounds(f.cu_q, b, f.total_q);
  const int row = cc / G, head = g * G + cc % G;
  if (cc >= G * (kDecCols / G) || row >= sq.len) return;
  const float* ml = a.part_ml + (size_t)grp * a.splits * (kDecCols * 2) + 2 * cc;  // split s at s * 64
  const float* po = a.part_o + (size_t)grp * a.splits * (kDecCols * kD) + cc * kD + d;  // split s at s * 2048
  const float sink2 = f.sinks[head] * kLog2e;
  float mm = sink2;
  for (int s = 0; s < a.splits; ++s) mm = fmaxf(mm, ml[s * (kDecCols * 2)]);
  float o = 0.f, l = 0.f;
  if (mm > -INFINITY) {
    l = sink2 > -INFINITY ? fast_exp2(sink2 - mm) : 0.f;  // the sink's mass, once
    for (int s = 0; s < a.splits; ++s) {
      const float ms = ml[s * (kDecCols * 2)];
      if (ms == -INFINITY) continue;  // a split that saw no key of this row
      const float sc = fast_exp2(ms - mm);
      o += po[(size_t)s * (kDecCols * kD)] * sc;
      l += ml[s * (kDecCols * 2) + 1] * sc;
    }
  }
  const size_t orow = (size_t)(sq.start + row) * f.hq + head;
  static_cast<T*>(f.o)[orow * kD + d] = from_f32<T>(l > 0.f ? o / l : 0.f);
  if (d == 0) f.lse[(size_t)head * f.total_q + sq.start + row] = l > 0.f ? (mm + fast_log2(l)) * kLn2 : -INFINITY;
}

bool decode_supported(int hq, int hkv, int max_q) { return (long long)(hq / hkv) * max_q <= kDecCols; }

DecodeWorkspace decode_workspace_layout(int hkv, int num_seqs, int max_q, int max_k, int window) {
  // Keys one sequence's rows can see, in tiles (a window may straddle one more tile).
  long long span = max_k;
  if (window > 0 && (long long)window + max_q - 1 < span) span = (long long)window + max_q - 1;
  const long long tiles = (span + kDecBN - 1) / kDecBN + (window > 0 ? 1 : 0);
  // About four workgroups per compute unit, each with at least one tile per wavefront.
  const long long groups = (long long)num_seqs * hkv;
  long long s = (1024 + groups - 1) / groups;
  const long long cap = (tiles + kDecWaves - 1) / kDecWaves;
  if (s > cap) s = cap;
  if (s > 65535) s = 65535;
  if (s < 1) s = 1;
  DecodeWorkspace w;
  w.splits = (int)s;
  const size_t parts = (size_t)groups * (size_t)s * kDecCols;
  w.part_o = 0;
  w.part_ml = (parts * kD * sizeof(float) + 255) & ~(size_t)255;
  w.total = w.part_ml + ((parts * 2 * sizeof(float) + 255) & ~(size_t)255);
  return w;
}

hipError_t launch_decode_partial(const DecodeArgs& a, int fp32, hipStream_t stream) {
  dim3 grid(a.f.num_seqs * a.f.hkv, a.splits);
  if (fp32)
    hipLaunchKernelGGL(decode_partial_kernel<float>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_partial_kernel<bf16>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeArgs& a, int fp32, hipStream_t stream) {
  dim3 grid(a.f.num_seqs * a.f.hkv, kDecCols / 4);
  if (fp32)
    hipLaunchKernelGGL(decode_merge_kernel<float>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_merge_kernel<bf16>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn_sink
