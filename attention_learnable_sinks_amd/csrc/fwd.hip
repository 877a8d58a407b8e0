// Forward of attention with per-head learnable sinks on gfx950.
//
// Computes, per query row i of head h (kv head g = h / (Hq/Hkv)),
//   o_i = sum_j P_ij v_j,  P_ij = exp(s_ij) / (sum_j' exp(s_ij') + exp(S_h)),
//   lse_i = log(sum_j exp(s_ij) + exp(S_h)),
// the sink softmax of "Unlocking Agentic RL Training for GPT-OSS" (euno.news),
// sub-sections 带汇聚的注意力 (sink logit appended to every score row, dropped
// before the product with V) and 数学公式 (the two probability formulas).
//
// Design (FlashAttention-style single pass, one workgroup per 128 query rows of
// one head; 4 wavefronts x 32 rows):
//   * Q stays in registers as the B operand of S^T = K Q^T, so each lane owns one
//     query row of S^T and all row reductions are in-lane (plus one lane-half swap).
//   * K and V tiles of 64 keys are double-buffered row-major in LDS, loaded straight
//     from HBM into LDS by buffer loads (swizzled so the operand reads are
//     conflict-free); the V^T operand of O^T = V^T P^T is read with transposing LDS
//     loads.  Operand addresses are per-lane registers plus immediates.
//   * Online softmax in the exp2 domain, P = exp2(fma(s, scale*log2e, -m)), with
//     the running max m seeded by the sink logit S_h*log2(e); the sink's own mass
//     exp2(S_h*log2e - m) is added once at the end.  m is not tracked per tile:
//     it only has to keep every P below 2^64 (exact either way, since m cancels in
//     O / l and lse = m + log2 l), so a tile is checked through the row sum it
//     produces anyway, and only a tile whose sum breaks the bound (or is inf / NaN,
//     as for S_h = -inf) takes the slow path: recompute its scores from the K tile
//     still in LDS, raise m to their max, rescale O and l, redo the exponentials.
//   * O^T = V^T P^T takes P (rounded to the element type) straight from the
//     registers of S^T as its B operand.
//   * Tiles outside the causal / sliding-window band are never visited; the mask
//     is evaluated only on tiles that straddle a band edge or the sequence end.
//   * Longest query tiles are dispatched first (causal load balance), and the
//     query heads that share a kv head are placed on one XCD so their K/V tiles
//     hit the same L2.
//   * Sliding-window layers pack the query heads of a kv head into the rows of a
//     tile (positions x heads): a tile then spans fewer positions and visits fewer
//     key tiles, and the heads share every K/V tile it loads.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace attn_sink {

// Bound on one lane's sum of exp2(x - m) over a key tile.  While every tile sum
// stays below it no probability exceeds 2^64, so P and the fp32 sums O and l
// cannot overflow for any realistic length and |v|.
constexpr float kTileSumMax = 18446744073709551616.f;  // 2^64

template <typename T, int D>
struct FwdCfg {
  static constexpr int BM = 128;       // query rows per workgroup
  static constexpr int BN = 64;        // keys per tile
  static constexpr int THREADS = 256;  // 4 wavefronts x 32 rows
  static constexpr int TILE = tile_elems_d<T, D>(BN);
  // bf16 at d = 64 runs four workgroups per compute unit (registers capped at 128),
  // one wavefront of each per SIMD, and raises its wavefront priority while it
  // issues MFMAs: a wavefront whose matrix work is ready goes first, and the
  // exponentials of the others fill the cycles the matrix core leaves to the
  // vector ALU.  The priority windows also bound how far the compiler hoists LDS
  // reads, which keeps the kernel inside 128 registers without spilling.  Measured
  // against three workgroups per compute unit without priority: 4k causal -0.5 to
  // -1%, 20k causal -1 to -4%, window-128 layers -5%.
  static constexpr bool PACKED = sizeof(T) == 2 && D == 64;
  static constexpr int MIN_WG = PACKED ? 4 : 1;
};

// D: head dim (64 or 128).
template <typename T, int D, bool PKH>
__global__ __launch_bounds__(256, (FwdCfg<T, D>::MIN_WG)) void fwd_kernel(FwdArgs p) {
  using C = FwdCfg<T, D>;
  using M = Mfma<T>;
  using Frag = typename M::Frag;
  constexpr int E = M::E, KS = M::KS;
  constexpr int NP = C::BN / KS;  // operand steps over the keys of a tile
  __shared__ __attribute__((aligned(16))) T smem[4 * C::TILE];  // [buf][K, V]

  // PKH (head-packed tiles, for sliding-window layers): the 128 rows of a tile are
  // BM / G query positions x the G query heads of one kv head, row r = position
  // r / G, head r % G.  A window tile then spans BM / G positions instead of BM, so
  // it visits fewer key tiles, and the G heads share each K/V tile it loads.
  // Packed: G divides BM, so it is a power of two (2^lg) and a row's position and
  // head are a shift and a mask.  The grid is (kv head, tile, sequence): in the
  // linear order the XCDs are dealt, kv head g lands on XCD g % 8 and each XCD
  // receives consecutive tiles of one sequence.  (Tile-major, one XCD receives one
  // workgroup per sequence in turn; where only the longest sequence still has tiles, the
  // working workgroups recur with the period of the batch size and the ragged batch above
  // ran 23% slower than per-head tiles.)  Per-head: longest causal tiles first.
  const int G = p.hq / p.hkv;
  const int lg = PKH ? __builtin_ctz(G) : 0;
  const XcdSlot slot = PKH ? XcdSlot{(int)blockIdx.z, (int)blockIdx.x, 0} : xcd_slot(blockIdx.x, p.hkv, G);
  const int bmq = PKH ? C::BM >> lg : C::BM;  // query positions per workgroup
  const int b = slot.seq, g = slot.kv;
  const int tile = PKH ? (int)blockIdx.y : gridDim.y - 1 - blockIdx.y;

  const SeqBounds sq = seq_bounds(p.cu_q, b, p.total_q);
  const SeqBounds sk = seq_bounds(p.cu_k, b, p.total_k);
  const int nq = sq.len, nk = sk.len, off = nk - nq;
  const int qs = tile * bmq;
  if (qs >= nq) return;
  const int qe = min(qs + bmq, nq);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront index (uniform)
  const int h = lane >> 5, c = lane & 31;
  const int head = PKH ? g * G + ((32 * w + c) & (G - 1)) : g * G + slot.item;  // this lane's row's head

  // Key range of the workgroup and of this wavefront.
  const int khi = p.causal ? clampi(qe - 1 + off + 1, 0, nk) : nk;
  const int klo = p.window > 0 ? clampi(qs + off - p.window + 1, 0, nk) : 0;
  const int qw = PKH ? qs + ((32 * w) >> lg) : qs + 32 * w;                    // first position of the wavefront
  const int qw_end = min(PKH ? qs + ((32 * w + 31) >> lg) + 1 : qw + 32, nq);  // one past its last
  const bool wave_rows = qw < nq;
  // Every row's keys form one interval [lo_i, hi_i) whose ends do not decrease with
  // the row: the wavefront's rows see keys in [wlo, whi) and all of them see
  // [wlo_all, whi_all).
  int whi = p.causal ? clampi(qw_end - 1 + off + 1, 0, nk) : nk;
  int wlo = p.window > 0 ? clampi(qw + off - p.window + 1, 0, nk) : 0;
  const int whi_all = p.causal ? clampi(qw + off + 1, 0, nk) : nk;
  const int wlo_all = p.window > 0 ? clampi(qw_end - 1 + off - p.window + 1, 0, nk) : 0;
  if (!wave_rows) whi = wlo = 0;

  const size_t kv_row = (size_t)p.hkv * D;
  const T* kbase_p = static_cast<const T*>(p.k) + (size_t)sk.start * kv_row + g * D;
  const T* vbase_p = static_cast<const T*>(p.v) + (size_t)sk.start * kv_row + g * D;

  // Q fragments (B operand of S^T = K Q^T): lane owns query qw + c, d = KS*s + E*h + e.
  const int qi = PKH ? qs + ((32 * w + c) >> lg) : qw + c;  // this lane's row's position
  typename M::Frag qf[D / KS];
  {
    const bool ok = qi < nq;
    const T* src = static_cast<const T*>(p.q) + ((size_t)(sq.start + (ok ? qi : 0)) * p.hq + head) * D;
#pragma unroll
    for (int s = 0; s < D / KS; ++s) qf[s] = global_frag<T>(src + KS * s + E * h, ok);
  }

  const float sink = p.sinks[head];
  const float sink2 = sink * kLog2e;
  const float sl2 = p.scale * kLog2e;
  float m_run = sink2;  // running max in the exp2 domain, seeded with the sink logit
  float l_run = 0.f;    // this lane's partial sum of exp2(x - m_run) over its keys
  f32x16 oacc[D / 32];  // O^T: [D x 32 rows]
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;

  const int kt_begin = klo / C::BN;
  const int kt_end = khi > klo ? (khi + C::BN - 1) / C::BN : kt_begin;

  const Span row_keys = keys_of_row(qi, off, nk, p.causal, p.window);  // the keys row qi sees
  FragAddr<T> fa;
  fa.init(lane, !C::PACKED);
  TileLoaderD<T, C::BN, C::THREADS, D> kld, vld;
  kld.init(kbase_p, kv_row, nk, tid);
  vld.init(vbase_p, kv_row, nk, tid);
  if (kt_begin < kt_end) {
    kld.issue_rebased(kt_begin * C::BN, smem);
    vld.issue_rebased(kt_begin * C::BN, smem + C::TILE);
    kld.finish();
    vld.finish();
  }
  vmem_drain();
  __syncthreads();

  // Which 32-key halves of the tile at kbase any row of the wavefront sees (bit mt
  // for keys kbase + 32 mt ..+32), and which of those every row sees in full; the
  // others need the per-element mask.  Wavefront-uniform.
  auto half_live = [&](int kbase) __attribute__((always_inline)) -> int {
    int live = 0;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int a = kbase + 32 * mt;
      live |= (a < whi && a + 32 > wlo) ? 1 << mt : 0;
    }
    return live;
  };
  auto half_full = [&](int kbase) __attribute__((always_inline)) -> int {
    int full = 0;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int a = kbase + 32 * mt;
      full |= (a >= wlo_all && a + 32 <= whi_all) ? 1 << mt : 0;
    }
    return full;
  };
  // S^T of one tile [64 keys x 32 queries].  Tiles that straddle a band edge are
  // masked to -inf outside the band, per 32-key half: halves every row sees take no
  // mask, halves no row sees none either (their probabilities are set to zero).
  auto scores = [&](f32x16* st, const T* Ks, int kbase, int live, auto full_tag) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    if constexpr (C::PACKED) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[mt][r] = 0.f;
#pragma unroll
      for (int s = 0; s < D / KS; ++s) st[mt] = M::mma(frag_row<T, C::BN>(fa, Ks, mt, s), qf[s], st[mt]);
    }
    if constexpr (C::PACKED) __builtin_amdgcn_s_setprio(0);
    if constexpr (!FULL) {
      const int full = half_full(kbase);
      // key of register r in tile mt: kbase + 4h + (32 mt + 8 (r/4) + r%4), a constant per element
      const int k0 = kbase + 4 * h;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        if ((live & ~full) >> mt & 1) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            st[mt][r] = in_span(k0 + 32 * mt + 8 * (r / 4) + r % 4, row_keys) ? st[mt][r] : -INFINITY;
        }
    }
  };
  // P = exp2(s * sl2 + neg_m) in place, rounded into operands; returns the lane's
  // sum of P in fp32, taken before the rounding.  The sum uses plain fp32 adds:
  // the bf16 dot-product instruction that could sum the rounded operands directly
  // does not overlap with the MFMAs of the other wavefronts on the SIMD, while
  // adds do (measured: about 0.15 against 0.55 overlap); about 1% faster here.
  auto probs = [&](f32x16* st, Frag* pf, float neg_m, int live, auto full_tag) __attribute__((always_inline)) -> float {
    constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      if (FULL || (live >> mt & 1)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) st[mt][r] = fast_exp2(fmaf(st[mt][r], sl2, neg_m));
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) st[mt][r] = 0.f;
      }
    }
    float sum = 0.f;
#pragma unroll
    for (int s = 0; s < NP; ++s) {
      if constexpr (sizeof(T) == 2) {
        const int r0 = 8 * (s % 2);
        const f32x16& x = st[s / 2];
        sum += ((x[r0] + x[r0 + 1]) + (x[r0 + 2] + x[r0 + 3])) + ((x[r0 + 4] + x[r0 + 5]) + (x[r0 + 6] + x[r0 + 7]));
        pf[s] = pack_frag<T>(st, s);
      } else {
        pf[s] = pack_frag<T>(st, s);
        sum = frag_sum<T>(pf[s], sum);
      }
    }
    return sum;
  };

  // One tile: S^T, (mask), P^T, O^T += V^T P^T.
  auto body = [&](const T* Ks, const T* Vs, int kbase, auto full_tag) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int live = FULL ? 3 : half_live(kbase);
    f32x16 st[2];
    Frag pf[NP];
    scores(st, Ks, kbase, live, full_tag);
    float tsum = probs(st, pf, -m_run, live, full_tag);  // m_run = -inf gives inf / NaN: caught below
    const bool over = !(tsum <= kTileSumMax);
    if (__any(over)) {
      // Slow path (rare): raise the running max to this tile's row max.  The K
      // tile is still in LDS, so the scores are simply computed again.  Only rows
      // whose own tile sum broke the bound change anything, so a row's result never
      // depends on the other rows of the wavefront (a row computed alone, e.g. one
      // decode step, comes out bitwise the same as in a full forward).
      const bool row_over = halves_max(over ? 1.f : 0.f) > 0.f;  // either half of the row
      scores(st, Ks, kbase, live, full_tag);
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        if (FULL || (live >> mt & 1)) {
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[mt][r]);
        }
      mx = halves_max(mx) * sl2;
      const float m_new = row_over ? fmaxf(m_run, mx) : m_run;
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);  // 0 when m_run = -inf
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;
      m_run = m_new;
      // m_new = -inf: every score of the row is masked so far, exp2(-inf + 0) = 0.
      tsum = probs(st, pf, m_new == -INFINITY ? 0.f : -m_new, live, full_tag);
    }
    l_run += tsum;
    // O^T[d x q] += V^T[d x keys] . P^T[keys x q]
    if constexpr (C::PACKED) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < NP; ++s)
#pragma unroll
      for (int md = 0; md < D / 32; ++md) oacc[md] = M::mma(frag_col<T, C::BN>(fa, Vs, md, s), pf[s], oacc[md]);
    if constexpr (C::PACKED) __builtin_amdgcn_s_setprio(0);
  };
  // One pipeline step: start loading tile kt+1 into the other buffer, compute tile
  // kt, wait for the load, barrier.  `cur` / `nxt` are the two buffers (K then V).
  auto step = [&](int kt, T* cur, T* nxt, auto full_tag) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    const bool more = kt + 1 < kt_end;
    if (more) {  // nxt was last read in the previous step, before its barrier
      kld.issue_rebased((kt + 1) * C::BN, nxt);
      vld.issue_rebased((kt + 1) * C::BN, nxt + C::TILE);
    }
    const int kbase = kt * C::BN;
    if constexpr (FULL) {
      body(cur, cur + C::TILE, kbase, full_tag);
    } else {
      if (kbase < whi && kbase + C::BN > wlo) body(cur, cur + C::TILE, kbase, full_tag);  // some half is live
    }
    if (more) {
      kld.finish();
      vld.finish();
    }
    __syncthreads();
  };
  T* const buf0 = smem;
  T* const buf1 = smem + 2 * C::TILE;
  auto masked_step = [&](int kt) __attribute__((always_inline)) {
    const bool odd = (kt - kt_begin) & 1;
    step(kt, odd ? buf1 : buf0, odd ? buf0 : buf1, std::false_type{});
  };
  // Tiles [wf_lo, wf_hi) are fully visible to every row of this wavefront: inside
  // the window's left edge, left of the diagonal and inside the sequence.  Every
  // wavefront runs the same number of steps (one barrier each), only the body
  // differs.  The unmasked tiles run in pairs so both buffer addresses are
  // compile-time constants there.
  int wf_lo = kt_begin, wf_hi = kt_begin;
  if (wave_rows) {
    const int lo_key = p.window > 0 ? qw_end + off - p.window : 0;  // first key every row sees from the left
    const int hi_key = p.causal ? min(qw + off + 1, nk) : nk;        // keys below this are seen by every row
    wf_lo = clampi(lo_key > 0 ? (lo_key + C::BN - 1) / C::BN : 0, kt_begin, kt_end);
    wf_hi = clampi(hi_key > 0 ? hi_key / C::BN : 0, wf_lo, kt_end);
  }
  int kt = kt_begin;
  for (; kt < wf_lo; ++kt) masked_step(kt);
  if (kt < wf_hi && ((kt - kt_begin) & 1)) {
    step(kt, buf1, buf0, std::true_type{});
    ++kt;
  }
  for (; kt + 1 < wf_hi; kt += 2) {
    step(kt, buf0, buf1, std::true_type{});
    step(kt + 1, buf1, buf0, std::true_type{});
  }
  if (kt < wf_hi) {
    step(kt, buf0, buf1, std::true_type{});
    ++kt;
  }
  for (; kt < kt_end; ++kt) masked_step(kt);

  // ---- epilogue: add the sink's mass once, normalise, write O and LSE.
  const float m_use = m_run == -INFINITY ? 0.f : m_run;
  float l_tot = halves_sum(l_run);
  if (sink2 > -INFINITY) l_tot += fast_exp2(sink2 - m_use);  // m_run >= sink2: at most 1
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qi < nq) {
    T* dst = static_cast<T*>(p.o) + ((size_t)(sq.start + qi) * p.hq + head) * D;
#pragma unroll
    for (int md = 0; md < D / 32; ++md)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * md + crow(4 * r4, h);
        if constexpr (sizeof(T) == 2) {
          bf16x4 v4 = {(bf16)(oacc[md][4 * r4] * inv), (bf16)(oacc[md][4 * r4 + 1] * inv),
                       (bf16)(oacc[md][4 * r4 + 2] * inv), (bf16)(oacc[md][4 * r4 + 3] * inv)};
          *reinterpret_cast<bf16x4*>(dst + d0) = v4;
        } else {
          f32x4 v4 = {oacc[md][4 * r4] * inv, oacc[md][4 * r4 + 1] * inv, oacc[md][4 * r4 + 2] * inv,
                      oacc[md][4 * r4 + 3] * inv};
          *reinterpret_cast<f32x4*>(dst + d0) = v4;
        }
      }
    if (h == 0)
      p.lse[(size_t)head * p.total_q + sq.start + qi] = l_tot > 0.f ? (m_use + fast_log2(l_tot)) * kLn2 : -INFINITY;
  }
}

// Head-packed tiles (they need G | BM and G > 1) on sliding-window layers.  A tile
// of BM positions visits about (BM + window) / BN key tiles, one of BM / G positions
// about (BM / G + window) / BN.  Measured at window 128, G = 8 (GPT-OSS shapes),
// against per-head tiles: one 16k sequence 105 against 115 us, eight of 6225 rows
// 318 against 362, the ragged batch of eight (1,277 to 14,090 rows) 336 against
// 369.  Both layouts give every row bitwise the same result: a row's arithmetic
// does not depend on the other rows of its tile.
static bool fwd_head_packed(const FwdArgs& a) {
  const int G = a.hq / a.hkv;
  if (a.window <= 0 || G < 2 || FwdCfg<bf16, 64>::BM % G != 0) return false;
  const long long tiles = ((long long)a.max_q * G + FwdCfg<bf16, 64>::BM - 1) / FwdCfg<bf16, 64>::BM;
  return tiles * a.num_seqs <= 65535;
}

template <typename T, int D>
static void launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  constexpr int BM = FwdCfg<T, D>::BM;
  if (fwd_head_packed(a)) {
    const int bmq = BM / (a.hq / a.hkv);
    dim3 grid(a.hkv, (a.max_q + bmq - 1) / bmq, a.num_seqs);
    hipLaunchKernelGGL((fwd_kernel<T, D, true>), grid, dim3(256), 0, stream, a);
  } else {
    dim3 grid(a.hq * a.num_seqs, (a.max_q + BM - 1) / BM);
    hipLaunchKernelGGL((fwd_kernel<T, D, false>), grid, dim3(256), 0, stream, a);
  }
}

hipError_t launch_fwd(const FwdArgs& a, int fp32, hipStream_t stream) {
  if (a.max_q == 0 || a.num_seqs == 0) return hipSuccess;
  if (a.d == 128) {
    if (fp32)
      launch_fwd_t<float, 128>(a, stream);
    else
      launch_fwd_t<bf16, 128>(a, stream);
  } else {
    if (fp32)
      launch_fwd_t<float, 64>(a, stream);
    else
      launch_fwd_t<bf16, 64>(a, stream);
  }
  return hipGetLastError();
}

}  // namespace attn_sink
