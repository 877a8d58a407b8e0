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
//     query row of S^T; row max / row sum are in-lane plus one lane-half swap.
//   * K and V tiles of 64 keys are double-buffered row-major in LDS, loaded straight
//     from HBM into LDS by buffer loads (swizzled so the operand reads are
//     conflict-free); the V^T operand of O^T = V^T P^T is read with transposing LDS
//     loads.
//   * Online softmax in the exp2 domain (exp2(fma(s, scale*log2e, -m))).  The running
//     max starts at the sink logit S_h*log2(e), not at -inf; the sink's own mass
//     exp2(S_h*log2e - m) is added once at the end.  The running max is only raised
//     (and O rescaled) when a row max exceeds it by more than 2^8, which after the
//     first tiles almost never happens.  S_h = -inf is standard attention: the
//     guarded max avoids exp2(-inf - -inf).
//   * O^T = V^T P^T reuses the S^T accumulator registers as the B operand (P
//     rounded to the element type), so P never leaves registers.
//   * Tiles outside the causal / sliding-window band are never visited; the mask
//     is evaluated only on tiles that straddle a band edge or the sequence end.
//   * Longest query tiles are dispatched first (causal load balance), and the
//     query heads that share a kv head are placed on one XCD so their K/V tiles
//     hit the same L2.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace attn_sink {

// Largest amount (log2 units) by which the running max may trail the row max.
constexpr float kSlack = 8.f;

template <typename T>
struct FwdCfg {
  static constexpr int BM = 128;       // query rows per workgroup
  static constexpr int BN = 64;        // keys per tile
  static constexpr int THREADS = 256;  // 4 wavefronts x 32 rows
  static constexpr int TILE = tile_elems<T>(BN);
};

template <typename T>
__global__ __launch_bounds__(256) void fwd_kernel(FwdArgs p) {
  using C = FwdCfg<T>;
  using M = Mfma<T>;
  constexpr int E = M::E, KS = M::KS;
  __shared__ __attribute__((aligned(16))) T smem[4 * C::TILE];  // [buf][K, V]

  const XcdSlot slot = xcd_slot(blockIdx.x, p.hkv, p.hq / p.hkv);
  const int b = slot.seq, g = slot.kv;
  const int head = g * (p.hq / p.hkv) + slot.item;
  const int tile = gridDim.y - 1 - blockIdx.y;  // longest causal tiles first

  const SeqBounds sq = seq_bounds(p.cu_q, b, p.total_q);
  const SeqBounds sk = seq_bounds(p.cu_k, b, p.total_k);
  const int nq = sq.len, nk = sk.len, off = nk - nq;
  const int qs = tile * C::BM;
  if (qs >= nq) return;
  const int qe = min(qs + C::BM, nq);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront index (uniform)
  const int h = lane >> 5, c = lane & 31;

  // Key range of the workgroup and of this wavefront.
  const int khi = p.causal ? clampi(qe - 1 + off + 1, 0, nk) : nk;
  const int klo = p.window > 0 ? clampi(qs + off - p.window + 1, 0, nk) : 0;
  const int qw = qs + 32 * w;
  const int qw_end = min(qw + 32, nq);
  const bool wave_rows = qw < nq;
  int whi = p.causal ? clampi(qw_end - 1 + off + 1, 0, nk) : nk;
  int wlo = p.window > 0 ? clampi(qw + off - p.window + 1, 0, nk) : 0;
  if (!wave_rows) whi = wlo = 0;

  const size_t kv_row = (size_t)p.hkv * kD;
  const T* kbase_p = static_cast<const T*>(p.k) + (size_t)sk.start * kv_row + g * kD;
  const T* vbase_p = static_cast<const T*>(p.v) + (size_t)sk.start * kv_row + g * kD;

  // Q fragments (B operand of S^T = K Q^T): lane owns query qw + c, d = KS*s + E*h + e.
  const int qi = qw + c;
  typename M::Frag qf[kD / KS];
  {
    const bool ok = qi < nq;
    const T* src = static_cast<const T*>(p.q) + ((size_t)(sq.start + (ok ? qi : 0)) * p.hq + head) * kD;
#pragma unroll
    for (int s = 0; s < kD / KS; ++s) qf[s] = global_frag<T>(src + KS * s + E * h, ok);
  }

  const float sink = p.sinks[head];
  const float sink2 = sink * kLog2e;
  const float sl2 = p.scale * kLog2e;
  float m_run = sink2;  // running max in the exp2 domain, seeded with the sink logit
  float l_run = 0.f;    // this lane's partial sum of exp2(x - m_run) over its keys
  f32x16 oacc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;

  const int kt_begin = klo / C::BN;
  const int kt_end = khi > klo ? (khi + C::BN - 1) / C::BN : kt_begin;

  TileLoader<T, C::BN, C::THREADS> kld, vld;
  kld.init(kbase_p, kv_row, nk, tid);
  vld.init(vbase_p, kv_row, nk, tid);
  if (kt_begin < kt_end) {
    kld.issue(kt_begin * C::BN, smem);
    vld.issue(kt_begin * C::BN, smem + C::TILE);
    kld.finish();
    vld.finish();
  }
  __syncthreads();

  // One tile: S^T, (mask), online softmax, O^T += V^T P^T.  FULL tiles need no mask;
  // the masked instantiation selects per element without branches.  Both are
  // straight-line code so the scheduler can overlap LDS reads, MFMA and exp.
  auto body = [&](const T* Ks, const T* Vs, int kbase, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    f32x16 sacc[2];  // S^T tile [64 keys x 32 queries] as two 32x32 tiles
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[mt][r] = 0.f;
#pragma unroll
      for (int s = 0; s < kD / KS; ++s)
        sacc[mt] = M::mma(lds_row_frag<T>(Ks, 32 * mt + c, KS * s + E * h), qf[s], sacc[mt]);
    }
    if constexpr (!FULL) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sacc[mt][r] =
              visible(qi, kbase + 32 * mt + crow(r, h), off, nk, p.causal, p.window) ? sacc[mt][r] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mt][r]);
    mx = halves_max(mx) * sl2;
    // Lazy rescale: the running max may trail the true max by up to kSlack (so
    // probabilities stay <= 2^kSlack); O and l are rescaled only when some row of
    // the wavefront exceeds that, which after the first tiles is rare.
    if (__any(mx > m_run + kSlack)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);  // 0 when m_run = -inf
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;
      m_run = m_new;
    }
    const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[mt][r] = fast_exp2(fmaf(sacc[mt][r], sl2, neg_m));
    // O^T[d x q] += V^T[d x keys] . P^T[keys x q]; the row sum is taken from the same
    // rounded P that multiplies V.
#pragma unroll
    for (int s = 0; s < C::BN / KS; ++s) {
      const typename M::Frag pf = pack_frag<T>(sacc, s);
      l_run = frag_sum<T>(pf, l_run);
#pragma unroll
      for (int md = 0; md < 2; ++md) oacc[md] = M::mma(lds_col_frag<T>(Vs, 32 * md, s, lane, true), pf, oacc[md]);
    }
  };
  // One pipeline step: prefetch tile kt+1 into registers, compute tile kt from LDS,
  // commit the prefetched tile to the other buffer, barrier.
  auto step = [&](int kt, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int buf = (kt - kt_begin) & 1;
    const bool more = kt + 1 < kt_end;
    T* nb = smem + (buf ^ 1) * 2 * C::TILE;  // read in the previous step, before its barrier
    if (more) {
      kld.issue((kt + 1) * C::BN, nb);
      vld.issue((kt + 1) * C::BN, nb + C::TILE);
    }
    const int kbase = kt * C::BN;
    const T* Ks = smem + buf * 2 * C::TILE;
    if constexpr (FULL) {
      body(Ks, Ks + C::TILE, kbase, full_tag);
    } else {
      if (kbase < whi && kbase + C::BN > wlo) body(Ks, Ks + C::TILE, kbase, full_tag);
    }
    if (more) {
      kld.finish();
      vld.finish();
    }
    __syncthreads();
  };
  // Tiles [wf_lo, wf_hi) are fully visible to every row of this wavefront: inside
  // the window's left edge, left of the diagonal and inside the sequence.  Every
  // wavefront runs the same number of steps (one barrier each), only the body differs.
  int wf_lo = kt_begin, wf_hi = kt_begin;
  if (wave_rows) {
    const int lo_key = p.window > 0 ? qw_end + off - p.window : 0;  // first key every row sees from the left
    const int hi_key = p.causal ? min(qw + off + 1, nk) : nk;        // keys below this are seen by every row
    wf_lo = clampi(lo_key > 0 ? (lo_key + C::BN - 1) / C::BN : 0, kt_begin, kt_end);
    wf_hi = clampi(hi_key > 0 ? hi_key / C::BN : 0, wf_lo, kt_end);
  }
  int kt = kt_begin;
  for (; kt < wf_lo; ++kt) step(kt, std::false_type{});
  for (; kt < wf_hi; ++kt) step(kt, std::true_type{});
  for (; kt < kt_end; ++kt) step(kt, std::false_type{});

  // ---- epilogue: add the sink's mass once, normalise, write O and LSE.
  const float m_use = m_run == -INFINITY ? 0.f : m_run;
  float l_tot = halves_sum(l_run);
  if (sink2 > -INFINITY) l_tot += fast_exp2(sink2 - m_use);  // m_run >= sink2: at most 1
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qi < nq) {
    T* dst = static_cast<T*>(p.o) + ((size_t)(sq.start + qi) * p.hq + head) * kD;
#pragma unroll
    for (int md = 0; md < 2; ++md)
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

hipError_t launch_fwd(const FwdArgs& a, int fp32, hipStream_t stream) {
  const int tiles = (a.max_q + FwdCfg<bf16>::BM - 1) / FwdCfg<bf16>::BM;
  if (tiles == 0 || a.num_seqs == 0) return hipSuccess;
  dim3 grid(a.hq * a.num_seqs, tiles);
  if (fp32)
    hipLaunchKernelGGL(fwd_kernel<float>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(fwd_kernel<bf16>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn_sink
