// Backward of attention with per-head learnable sinks on gfx950.
//
// The sink gradient is the one of "Unlocking Agentic RL Training for GPT-OSS"
// (euno.news), sub-section 反向传播, with the inner factor read as dL/dP_ij:
//   dS_h = -sum_i P_sink_i D_i,   D_i = sum_j P_ij dP_ij = <dO_i, O_i>,
//   P_sink_i = exp(S_h - lse_i).
// dq, dk, dv follow from the chain rule through the softmax over the score row
// with the sink column appended (the sink column gets no upstream gradient):
//   dP_ij = <dO_i, v_j>,  dS_ij = P_ij (dP_ij - D_i),
//   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,  dv_j = sum_i P_ij dO_i.
// P is recomputed from the forward's lse (which includes the sink), so the sink
// needs no other state in the backward.
//
// Three kernels on one stream, none using atomics, so every output is bitwise
// reproducible:
//   1. bwd_dq:     query-stationary (like the forward): D_i = <dO_i, O_i> from the
//                  row's own O and dO fragments, the row statistics (lse * log2 e,
//                  -D) for the dK/dV kernel and a per-workgroup partial sum of
//                  -P_sink_i D_i; then per 64-key tile S^T = K Q^T, dP^T = V dO^T,
//                  dQ^T += K^T dS^T, with Q and dO in registers and K^T read from
//                  the row-major K tile by transposing LDS loads.  dQ is written
//                  once, scaled, in the element type.
//   2. bwd_dkdv:   key-stationary: a workgroup owns 128 keys of one kv head (32 per
//                  wavefront, K and V in registers) and loops over the query heads of
//                  its share of the GQA group and over the query tiles of the band
//                  (per-head tiles from the last down, so that the workgroups sharing
//                  a head's Q and dO read the same rows together):
//                  S = Q K^T, dP = dO V^T put the key on the lane, so P and dS feed
//                  dV^T += dO^T P and dK^T += Q^T dS from registers, with dO^T and Q^T
//                  read transposed from row-major LDS tiles.  Under a causal mask key
//                  tiles kt and n-1-kt are folded into one workgroup so all workgroups
//                  carry the same work.  When the group is split over several
//                  workgroups (to fill the GPU), each split writes an fp32 partial.
//   3. bwd_finish: fixed-order sums of the dS_h partials and of the dK/dV partials.
#include <type_traits>
#include <utility>

#include "common.h"
#include "kernels.h"

namespace attn_sink {

// ----------------------------------------------------------------------------- 1. dQ
template <typename T, int D>
struct DqCfg {
  static constexpr int BM = kDqRows;  // query rows per workgroup (4 wavefronts x 32)
  static constexpr int BN = 64;   // keys per tile
  static constexpr int THREADS = 256;
  static constexpr int TILE = tile_elems_d<T, D>(BN);
  // Workgroups resident per compute unit the register budget is set for: three at
  // bf16 d = 64 (168 registers), two at bf16 d = 128; fp32 is left to the compiler.
  static constexpr int MIN_WG = sizeof(T) == 2 ? (D == 64 ? 3 : 2) : 1;
};

template <typename T, int D, bool PKH>
__global__ __launch_bounds__(256, (DqCfg<T, D>::MIN_WG)) void bwd_dq_kernel(BwdArgs a) {
  using C = DqCfg<T, D>;
  using M = Mfma<T>;
  constexpr int E = M::E, KS = M::KS;
  const FwdArgs& f = a.f;
  __shared__ __attribute__((aligned(16))) T smem[4 * C::TILE];  // [buf][K, V]
  __shared__ float red[PKH ? C::BM : 4];

  // PKH (head-packed tiles, sliding-window layers): the 128 rows of a tile are
  // BM / G positions x the G query heads of one kv head (row r: position r >> lg,
  // head r & (G - 1), G = 2^lg since it divides BM), as in the forward; the grid is
  // (kv head, tile, sequence).
  const int G = f.hq / f.hkv;
  const int lg = PKH ? __builtin_ctz(G) : 0;
  const XcdSlot slot = PKH ? XcdSlot{(int)blockIdx.z, (int)blockIdx.x, 0} : xcd_slot(blockIdx.x, f.hkv, G);
  const int bmq = PKH ? C::BM >> lg : C::BM;  // query positions per workgroup
  const int ntiles = (int)gridDim.y;           // row tiles per sequence
  const int b = slot.seq, g = slot.kv;
  const int tile = PKH ? (int)blockIdx.y : gridDim.y - 1 - blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront index (uniform)
  const int h = lane >> 5, c = lane & 31;
  const int head = PKH ? g * G + ((32 * w + c) & (G - 1)) : g * G + slot.item;  // this lane's row's head
  const SeqBounds sq = seq_bounds(f.cu_q, b, f.total_q);
  const SeqBounds sk = seq_bounds(f.cu_k, b, f.total_k);
  const int nq = sq.len, nk = sk.len, off = nk - nq;
  const int qs = tile * bmq;
  // This workgroup's slot of the dS_h partials (one per head, sequence and row tile);
  // packed: head g*G + j's slot is dsink_slot + j * pre_blocks.
  float* const dsink_slot =
      a.dsink_part + (size_t)(PKH ? g * G : head) * a.pre_blocks + (size_t)b * ntiles + tile;
  if (qs >= nq) {
    if (PKH ? tid < G : tid == 0) dsink_slot[(size_t)tid * a.pre_blocks] = 0.f;
    return;
  }
  const int qe = min(qs + bmq, nq);

  FragAddr<T> fa;
  fa.init(lane);
  const int khi = f.causal ? clampi(qe - 1 + off + 1, 0, nk) : nk;
  const int klo = f.window > 0 ? clampi(qs + off - f.window + 1, 0, nk) : 0;
  const int qw = PKH ? qs + ((32 * w) >> lg) : qs + 32 * w;        // first position of the wavefront
  const int qw_last = PKH ? qs + ((32 * w + 31) >> lg) : qw + 31;  // its last position
  const int qw_end = min(qw_last + 1, nq);
  // The wavefront's rows see keys in [wlo, whi); all of them see [wlo_all, whi_all)
  // (both ends of a row's key interval are nondecreasing in the row).
  int whi = f.causal ? clampi(qw_end - 1 + off + 1, 0, nk) : nk;
  int wlo = f.window > 0 ? clampi(qw + off - f.window + 1, 0, nk) : 0;
  const int whi_all = f.causal ? clampi(qw + off + 1, 0, nk) : nk;
  const int wlo_all = f.window > 0 ? clampi(qw_end - 1 + off - f.window + 1, 0, nk) : 0;
  if (qw >= nq) whi = wlo = 0;

  const size_t kv_row = (size_t)f.hkv * D, q_row = (size_t)f.hq * D;
  const T* kbase_p = static_cast<const T*>(f.k) + (size_t)sk.start * kv_row + g * D;
  const T* vbase_p = static_cast<const T*>(f.v) + (size_t)sk.start * kv_row + g * D;

  // Q and dO fragments (B operands of S^T = K Q^T and dP^T = V dO^T); lse and D of the lane's row.
  const int qi = PKH ? qs + ((32 * w + c) >> lg) : qw + c;  // this lane's row's position
  const bool qok = qi < nq;
  Span row_keys = keys_of_row(qi, off, nk, f.causal, f.window);  // the keys row qi sees
  if (!qok) row_keys.len = 0u;
  // Q, dO and O fragments of the lane's row (lane half h holds half of it); O only
  // for D_i = <dO_i, O_i>.
  typename M::Frag qf[D / KS], dof[D / KS], of[D / KS];
  {
    const size_t o = ((size_t)(sq.start + (qok ? qi : 0)) * f.hq + head) * D;
    const T* qsrc = static_cast<const T*>(f.q) + o;
    const T* dsrc = static_cast<const T*>(a.dout) + o;
    const T* osrc = static_cast<const T*>(f.o) + o;
#pragma unroll
    for (int s = 0; s < D / KS; ++s) {
      qf[s] = global_frag<T>(qsrc + KS * s + E * h, qok);
      dof[s] = global_frag<T>(dsrc + KS * s + E * h, qok);
      of[s] = global_frag<T>(osrc + KS * s + E * h, qok);
    }
  }
  const float lse = qok ? f.lse[(size_t)head * f.total_q + sq.start + qi] : 0.f;

  f32x16 dqt[D / 32];  // dQ^T [D x 32 q]
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqt[t][r] = 0.f;

  // The first K/V tile is in flight while the row statistics are formed.
  const int kt_begin = klo / C::BN;
  const int kt_end = khi > klo ? (khi + C::BN - 1) / C::BN : kt_begin;
  TileLoaderD<T, C::BN, C::THREADS, D> kld, vld;
  kld.init(kbase_p, kv_row, nk, tid);
  vld.init(vbase_p, kv_row, nk, tid);
  if (kt_begin < kt_end) {
    kld.issue_rebased(kt_begin * C::BN, smem);
    vld.issue_rebased(kt_begin * C::BN, smem + C::TILE);
    kld.finish();
    vld.finish();
  }
  float dpart = 0.f;
#pragma unroll
  for (int s = 0; s < D / KS; ++s) dpart = frag_dot<T>(of[s], dof[s], dpart);
  const float dd = halves_sum(dpart);  // D of the lane's row (0 past the sequence)
  const float lse2 = lse * kLog2e;
  const float sl2 = f.scale * kLog2e;
  // Row statistics for the dK/dV kernel: -lse * log2(e) (the seed of its score
  // accumulator) and -D (the seed of its dP accumulator).
  const bool writer = qok && h == 0;
  if (writer) {
    a.rowstat[(size_t)(2 * head) * f.total_q + sq.start + qi] = -lse2;
    a.rowstat[(size_t)(2 * head + 1) * f.total_q + sq.start + qi] = -dd;
  }
  // This lane's float32 sum of dS_ij = P_ij (dP_ij - D_i) over its keys (see the epilogue).
  float dsum = 0.f;
  f32x16 neg_dd;  // -D of the lane's row in every register
#pragma unroll
  for (int r = 0; r < 16; ++r) neg_dd[r] = -dd;
  vmem_drain();
  __syncthreads();

  // One tile: S^T, dP^T, P^T, dS^T, dQ^T += K^T dS^T.  FULL tiles need no mask; in
  // the others only the 32-key halves that not every row of the wavefront sees in
  // full take the per-element mask.
  auto body = [&](const T* Ks, const T* Vs, int kbase, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    int masked = 0;  // bit mt: keys kbase + 32 mt ..+32
    if constexpr (!FULL) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int k = kbase + 32 * mt;
        masked |= (k >= wlo_all && k + 32 <= whi_all) ? 0 : 1 << mt;
      }
    }
    // S^T, dP^T of the 32 keys kbase + 32 mt ..+32 against the wavefront's 32 rows.
    auto scores = [&](int mt, f32x16& st_out, f32x16& dpt_out) {
      f32x16 st, dpt;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        st[r] = 0.f;
        dpt[r] = 0.f;
      }
#pragma unroll
      for (int s = 0; s < D / KS; ++s) {
        st = M::mma(frag_row<T, C::BN>(fa, Ks, mt, s), qf[s], st);
        const auto vfr = frag_row<T, C::BN>(fa, Vs, mt, s);
        if constexpr (sizeof(T) == 2) {
          // bf16: dP^T starts from -D (a loop-invariant seed), so it ends at dP^T - D.
          dpt = s == 0 ? mma_seeded(vfr, dof[s], neg_dd) : M::mma(vfr, dof[s], dpt);
        } else {
          dpt = M::mma(vfr, dof[s], dpt);
        }
      }
      st_out = st;
      dpt_out = dpt;
    };
    // S^T -> P^T -> dS^T = P^T (dP^T - D) in place; returns the half's sum of dS^T.
    auto grads = [&](int mt, f32x16& st, const f32x16& dpt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[r] = fast_exp2(fmaf(st[r], sl2, -lse2));  // P^T
      if (!FULL && (masked >> mt & 1)) {
#pragma unroll
        for (int r = 0; r < 16; ++r)  // key kbase + 4h + (32 mt + 8 (r/4) + r%4)
          st[r] = in_span(kbase + 4 * h + 32 * mt + 8 * (r / 4) + r % 4, row_keys) ? st[r] : 0.f;
      }
      float t = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        st[r] *= sizeof(T) == 2 ? dpt[r] : dpt[r] - dd;
        t = r == 0 ? st[r] : t + st[r];
      }
      return t;
    };
    // dQ^T[d x q] += K^T[d x keys] . dS^T[keys x q] over contraction steps s0 ..+ns of
    // the tile, with dS^T held from step s0 on in st.
    auto dq_update = [&](const f32x16* st, int s0, auto ns_tag) {
      constexpr int NS = decltype(ns_tag)::value;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const typename M::Frag sf = pack_frag<T>(st, s);
#pragma unroll
        for (int md = 0; md < D / 32; ++md)
          dqt[md] = M::mma(frag_col<T, C::BN>(fa, Ks, md, s0 + s), sf, dqt[md]);
      }
    };
    constexpr int NS = C::BN / KS;  // dQ contraction steps per tile
    // Issue priority is raised while this wavefront feeds the matrix cores, so the
    // other wavefronts on the SIMD fill the vector ALUs meanwhile (measured faster).
    float tsum[2];  // the tile's row sums of dS^T, one chain per 32 keys
    if constexpr (D == 64) {
      // One 32-key half at a time: only one half's scores are live, which keeps
      // the kernel at its register cap without spills.  Same products, same order.
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x16 st, dpt;
        __builtin_amdgcn_s_setprio(1);
        scores(mt, st, dpt);
        __builtin_amdgcn_s_setprio(0);
        tsum[mt] = grads(mt, st, dpt);
        __builtin_amdgcn_s_setprio(1);
        dq_update(&st, mt * (NS / 2), std::integral_constant<int, NS / 2>{});
        __builtin_amdgcn_s_setprio(0);
      }
    } else {
      // Both halves' scores first: at D = 128 the by-halves form spills (bf16) or needs
      // more registers (fp32, 471 against 395).
      f32x16 st[2], dpt[2];
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) scores(mt, st[mt], dpt[mt]);
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) tsum[mt] = grads(mt, st[mt], dpt[mt]);
      __builtin_amdgcn_s_setprio(1);
      dq_update(st, 0, std::integral_constant<int, NS>{});
      __builtin_amdgcn_s_setprio(0);
    }
    dsum += tsum[0] + tsum[1];
  };
  auto step = [&](int kt, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int buf = (kt - kt_begin) & 1;
    const bool more = kt + 1 < kt_end;
    T* nb = smem + (buf ^ 1) * 2 * C::TILE;  // read in the previous step, before its barrier
    if (more) {
      kld.issue_rebased((kt + 1) * C::BN, nb);
      vld.issue_rebased((kt + 1) * C::BN, nb + C::TILE);
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
  // Tiles [wf_lo, wf_hi) are fully visible to all 32 rows of this wavefront.
  int wf_lo = kt_begin, wf_hi = kt_begin;
  if (qw_last < nq) {
    const int lo_key = f.window > 0 ? qw_end + off - f.window : 0;
    const int hi_key = f.causal ? min(qw + off + 1, nk) : nk;
    wf_lo = clampi(lo_key > 0 ? (lo_key + C::BN - 1) / C::BN : 0, kt_begin, kt_end);
    wf_hi = clampi(hi_key > 0 ? hi_key / C::BN : 0, wf_lo, kt_end);
  }
  int kt = kt_begin;
  for (; kt < wf_lo; ++kt) step(kt, std::false_type{});
  for (; kt < wf_hi; ++kt) step(kt, std::true_type{});
  for (; kt < kt_end; ++kt) step(kt, std::false_type{});

  // This workgroup's share of dS_h = -sum_i P_sink_i D_i.  D_i = sum_j P_ij dP_ij
  // is taken from the float32 P and dP of the loop, not from <dO_i, O_i> with O
  // rounded to the element type: a head whose dS_h is a near cancellation of its
  // rows' terms (large sinks over long rows) would otherwise carry that rounding
  // (about 2^-9 of each D_i) into a result many times smaller than the terms.
  // The loop summed dS_ij = P_ij (dP_ij - D'_i), D' = <dO_i, O_i>, so
  //   D_i = sum_j dS_ij + D'_i sum_j P_ij = sum_j dS_ij + D'_i (1 - P_sink_i).
  // Fixed-order reduction: lanes, then wavefronts (packed tiles: rows per head).
  {
    // (P_sink_i and D'_i are formed again here rather than held through the loop.)
    const float lse_e = qok ? f.lse[(size_t)head * f.total_q + sq.start + qi] : 0.f;
    const float sink = f.sinks[head];
    const bool wr = qok && h == 0;
    const float ps = (wr && lse_e > -INFINITY && sink > -INFINITY) ? fast_exp2((sink - lse_e) * kLog2e) : 0.f;
    const float d_row = halves_sum(dsum) - neg_dd[0] * (1.f - ps);
    float contrib = wr ? -ps * d_row : 0.f;
    if constexpr (PKH) {
      if (h == 0) red[32 * w + c] = contrib;  // by row; summed per head below
    } else {
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) contrib += __shfl_xor(contrib, m);
      if (lane == 0) red[w] = contrib;
    }
    __syncthreads();
    if constexpr (PKH) {
      // head g*G + tid: its rows tid, tid + G, ... in order
      if (tid < G) {
        float acc = 0.f;
        for (int r = tid; r < C::BM; r += G) acc += red[r];
        dsink_slot[(size_t)tid * a.pre_blocks] = acc;
      }
    } else {
      if (tid == 0) *dsink_slot = (red[0] + red[1]) + (red[2] + red[3]);
    }
  }

  if (qok) {
    T* dst = static_cast<T*>(a.dq) + (size_t)(sq.start + qi) * q_row + head * D;
#pragma unroll
    for (int md = 0; md < D / 32; ++md)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * md + crow(4 * r4, h);
        const f32x16& t = dqt[md];
        if constexpr (sizeof(T) == 2) {
          bf16x4 v4 = {(bf16)(t[4 * r4] * f.scale), (bf16)(t[4 * r4 + 1] * f.scale), (bf16)(t[4 * r4 + 2] * f.scale),
                       (bf16)(t[4 * r4 + 3] * f.scale)};
          *reinterpret_cast<bf16x4*>(dst + d0) = v4;
        } else {
          f32x4 v4 = {t[4 * r4] * f.scale, t[4 * r4 + 1] * f.scale, t[4 * r4 + 2] * f.scale, t[4 * r4 + 3] * f.scale};
          *reinterpret_cast<f32x4*>(dst + d0) = v4;
        }
      }
  }
}

// ----------------------------------------------------------------------------- 2. dK, dV
template <typename T, int D>
struct DkvCfg {
  static constexpr int BMB = 64;       // queries per tile
  static constexpr int THREADS = 256;  // 4 wavefronts
  static constexpr int BNB = kDkvKeys;  // keys per key tile (32 per wavefront)
  static constexpr int TILE = tile_elems_d<T, D>(BMB);
  // workgroups resident per compute unit (bf16 at d = 64 fits two; the others one)
  static constexpr int PER_CU = (sizeof(T) == 2 && D == 64) ? 2 : 1;
};

// PKH (head-packed query tiles, window layers, bf16, G = 8 query heads per kv head,
// one head split): the 64 rows of a query tile are 8 positions x the 8 query heads
// of the kv head (row r: position r >> 3, head r & 7), so a tile spans 8 positions
// instead of 64.  A wavefront's 32 keys are seen by about window + 31 positions;
// per-head 64-row tiles cover them with 3-4 tiles per head (1.2-1.6x the rows),
// packed tiles with whole 8-position steps (about 1.05x), most of them fully
// visible (no mask).  The rows of one position are one contiguous run of
// 8 x D elements in Q and dO.
template <typename T, int D, bool PKH>
__global__ __launch_bounds__((DkvCfg<T, D>::THREADS), (sizeof(T) == 2 && D == 64) ? 2 : 1) void bwd_dkdv_kernel(
    BwdArgs a) {
  static_assert(!PKH || sizeof(T) == 2, "head-packed dK/dV tiles are built for bf16");
  using C = DkvCfg<T, D>;
  using M = Mfma<T>;
  constexpr int E = M::E, KS = M::KS;
  const FwdArgs& f = a.f;
  // bf16 stages tiles two steps ahead (three buffers); fp32 stages through registers, one ahead.
  constexpr int NB = sizeof(T) == 2 ? 3 : 2;
  using QLoader = TileLoaderD<T, C::BMB, C::THREADS, D>;
  // bf16: this wavefront's DMA instructions per staged tile (Q and dO; waves 0 and 1
  // add one row-statistics load), for the waits in step().
  constexpr int kStageVm = 2 * QLoader::N;
  __shared__ __attribute__((aligned(16))) T smem[NB * 2 * C::TILE];  // [buf][Q, dO]
  __shared__ __attribute__((aligned(16))) float nlse_s[NB][C::BMB];  // -lse * log2(e) of the tile's rows
  __shared__ __attribute__((aligned(16))) float dd_s[NB][C::BMB];

  const XcdSlot slot = xcd_slot(blockIdx.x, f.hkv, a.splits);
  // Several sequences: blockIdx.y = sequence x its folded pairs (sequence-major), so the
  // workgroups one XCD receives are consecutive pairs of one sequence (the launcher then
  // leaves the sequences out of the x dimension).
  const int nfold = ((f.max_k + C::BNB - 1) / C::BNB + 1) / 2;
  const bool seq_major = f.num_seqs > 1 && (int)gridDim.x == f.hkv * a.splits;
  const int b = seq_major ? (int)blockIdx.y / nfold : slot.seq, g = slot.kv, split = slot.item;
  const int hps = (f.hq / f.hkv) / a.splits;  // query heads per split (PKH: all 8, one split)
  constexpr int TP = PKH ? C::BMB >> 3 : C::BMB;  // query positions per tile
  const int head0 = g * (f.hq / f.hkv) + split * hps;

  const SeqBounds sq = seq_bounds(f.cu_q, b, f.total_q);
  const SeqBounds sk = seq_bounds(f.cu_k, b, f.total_k);
  const int nq = sq.len, nk = sk.len, off = nk - nq;
  const int nkt = (nk + C::BNB - 1) / C::BNB;
  const int fold = seq_major ? (int)blockIdx.y % nfold : (int)blockIdx.y;
  if (fold >= (nkt + 1) / 2) return;
  // Two workgroups share a compute unit here, and the wavefront arbiter favours the older
  // one, which runs about a quarter faster; the pair then ends apart and the later one
  // runs alone. Workgroups of the second half of the grid (the younger of each pair)
  // raise their wavefront priority on two steps of every three to even the two out.
  const bool young = DkvCfg<T, D>::PER_CU == 2 && 2 * fold >= nfold;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront index (uniform)
  const int h = lane >> 5, c = lane & 31;
  FragAddr<T> fa;
  fa.init(lane);
  const size_t kv_row = (size_t)f.hkv * D, q_row = (size_t)f.hq * D;
  const float sl2 = f.scale * kLog2e;
  const T* qhead_p = static_cast<const T*>(f.q) + (size_t)sq.start * q_row;
  const T* dohead_p = static_cast<const T*>(a.dout) + (size_t)sq.start * q_row;

  const int n_phase = (nkt - 1 - fold != fold) ? 2 : 1;
  for (int phase = 0; phase < n_phase; ++phase) {
    const int kt = phase == 0 ? fold : nkt - 1 - fold;
    const int kbase = kt * C::BNB;
    const int kend = min(kbase + C::BNB, nk);
    const int qlo = f.causal ? clampi(kbase - off, 0, nq) : 0;
    const int qhi = f.window > 0 ? clampi(kend - 1 - off + f.window, 0, nq) : nq;
    const int qt_begin = qlo / TP;
    const int nqt = qhi > qlo ? (qhi + TP - 1) / TP - qt_begin : 0;
    const int n_it = PKH ? nqt : hps * nqt;

    const int kw = kbase + 32 * w;
    const int kw_end = min(kw + 32, nk);
    const bool wave_keys = kw < nk;
    const int wqlo = f.causal ? clampi(kw - off, 0, nq) : 0;
    const int wqhi = f.window > 0 ? clampi(kw_end - 1 - off + f.window, 0, nq) : nq;

    // K and V fragments (B operands of S = Q K^T and dP = dO V^T): lane owns key kj.
    const int kj = kw + c;
    const bool kok = kj < nk;
    const Span key_rows = rows_of_key(kj, off, nq, nk, f.causal, f.window);  // the rows that see key kj
    typename M::Frag kf[D / KS], vf[D / KS];
    {
      const size_t o = (size_t)(sk.start + (kok ? kj : 0)) * kv_row + g * D;
      const T* ksrc = static_cast<const T*>(f.k) + o;
      const T* vsrc = static_cast<const T*>(f.v) + o;
#pragma unroll
      for (int s = 0; s < D / KS; ++s) {
        kf[s] = global_frag<T>(ksrc + KS * s + E * h, kok);
        vf[s] = global_frag<T>(vsrc + KS * s + E * h, kok);
      }
    }

    f32x16 dkt[D / 32], dvt[D / 32];  // dK^T, dV^T: [D x 32 keys]
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dkt[t][r] = 0.f;
        dvt[t][r] = 0.f;
      }

    QLoader qld, dold;
    RowLoader lld, dld;  // the tile's lse * log2(e) and -D rows (waves 0 and 1)
    int staged_head = -1;
    if constexpr (PKH) {
      // One set of descriptors for the whole loop.  The row statistics of head
      // head0 + j sit 2 total_q apart; rows past the sequence read the next
      // sequence's (finite) statistics or zero past the array, and only ever meet
      // masked (zero) probabilities.
      qld.init_rows(qhead_p + head0 * D, q_row, nq, tid, 3, D * sizeof(T));
      dold.init_rows(dohead_p + head0 * D, q_row, nq, tid, 3, D * sizeof(T));
      const long long stat0 = (long long)(2 * head0) * f.total_q + sq.start;
      const int nstat = (int)((long long)2 * f.hq * f.total_q - stat0);
      lld.init_packed(a.rowstat + stat0, nstat);
      dld.init_packed(a.rowstat + stat0 + f.total_q, nstat - f.total_q);
    }
    // The next (head, query tile) to stage: stage() is called for iterations 0, 1, 2, ...
    // in order, so it advances a counter instead of dividing the iteration index.
    // Per-head tiles walk the query tiles from the last down.  Causal key tiles all see
    // the rows from their own up to the end of the sequence, so the workgroups that
    // share a head's Q and dO then read the same rows at about the same time, and the
    // L2 serves the re-reads.  (Packed tiles only run window layers, whose ranges
    // overlap between neighbouring key tiles alone; they walk upwards.)
    constexpr bool DOWN = !PKH;
    const int qt_first = DOWN ? qt_begin + nqt - 1 : qt_begin;
    int st_hd = head0, st_qt = qt_first;
    // Start moving (head, query tile) of iteration `it` into LDS buffer `buf`.
    auto stage = [&](int it, int buf) __device__ {
      if constexpr (PKH) {
        const int qt = qt_begin + it;
        qld.issue(qt * TP, smem + buf * 2 * C::TILE);
        dold.issue(qt * TP, smem + buf * 2 * C::TILE + C::TILE);
        if (w == 0) lld.issue_packed(qt * TP, nlse_s[buf], lane, 3, 2 * f.total_q);
        if (w == 1) dld.issue_packed(qt * TP, dd_s[buf], lane, 3, 2 * f.total_q);
        return;
      }
      const int hd = st_hd, qt = st_qt;
      if (DOWN ? --st_qt < qt_begin : ++st_qt == qt_begin + nqt) {
        st_qt = qt_first;
        ++st_hd;
      }
      if (hd != staged_head) {  // uniform: new descriptors when the query head changes
        qld.init(qhead_p + hd * D, q_row, nq, tid);
        dold.init(dohead_p + hd * D, q_row, nq, tid);
        lld.init(a.rowstat + (size_t)(2 * hd) * f.total_q + sq.start, nq);
        dld.init(a.rowstat + (size_t)(2 * hd + 1) * f.total_q + sq.start, nq);
        staged_head = hd;
      }
      qld.issue(qt * C::BMB, smem + buf * 2 * C::TILE);
      dold.issue(qt * C::BMB, smem + buf * 2 * C::TILE + C::TILE);
      // The row statistics go straight to LDS as well (rows past the sequence read
      // as 0), so no load in the loop writes a register the loop has to wait for.
      if (w == 0) lld.issue(qt * C::BMB, nlse_s[buf], lane);
      if (w == 1) dld.issue(qt * C::BMB, dd_s[buf], lane);
    };
    auto commit = [&](int buf) __device__ {
      qld.finish();
      dold.finish();  // also covers the row loads (same counter)
      (void)buf;
    };

    if (n_it > 0) {
      stage(0, 0);
      if constexpr (NB == 3) {
        if (n_it > 1) stage(1, 1);
      } else {
        commit(0);
      }
    }
    vmem_drain();
    __syncthreads();
    // One (head, query tile): S, dP, P, dS, dV^T += dO^T P, dK^T += Q^T dS.
    auto body = [&](int buf, int qbase, auto full_tag) __device__ {
      constexpr bool FULL = decltype(full_tag)::value;
      const T* Qs = smem + buf * 2 * C::TILE;
      const T* dOs = Qs + C::TILE;
      f32x16 pt[2], dst[2];  // P, dS: [64 q x 32 keys], key on the lane
#pragma unroll
      for (int mq = 0; mq < 2; ++mq) {
#pragma unroll
        for (int r = 0; r < 16; ++r) pt[mq][r] = 0.f;
        // -D of each register's query row (dd_s holds -D): the seed of the dP
        // accumulator, which then ends at dP - D.
        f32x16 seed;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&dd_s[buf][32 * mq + crow(4 * r4, h)]);
#pragma unroll
          for (int e = 0; e < 4; ++e) seed[4 * r4 + e] = d4[e];
        }
        // All operands of this block's 8 MFMAs are read first; the scheduling barrier
        // keeps the reads from being sunk next to their MFMAs (which would expose the
        // LDS latency once per MFMA).
        typename M::Frag qa[D / KS], da[D / KS];
#pragma unroll
        for (int s = 0; s < D / KS; ++s) {
          qa[s] = frag_row<T, C::BMB>(fa, Qs, mq, s);
          da[s] = frag_row<T, C::BMB>(fa, dOs, mq, s);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < D / KS; ++s) {
          pt[mq] = M::mma(qa[s], kf[s], pt[mq]);
          dst[mq] = s == 0 ? mma_first<T>(da[s], vf[s], seed) : M::mma(da[s], vf[s], dst[mq]);
        }
      }
#pragma unroll
      for (int mq = 0; mq < 2; ++mq)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int ql = 32 * mq + crow(4 * r4, h);  // 4 consecutive query rows
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&nlse_s[buf][ql]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * r4 + e;
            float pv = fast_exp2(fmaf(pt[mq][r], sl2, l4[e]));  // nlse_s holds -lse * log2(e)
            if constexpr (!FULL) {
              // tile row 4h + 32 mq + 8 r4 + e: per-head tiles, query qbase + that row;
              // packed, position qbase + 4 mq + r4 (the row >> 3), a constant per element
              const int qrow = PKH ? qbase + 4 * mq + r4 : qbase + 4 * h + 32 * mq + 8 * r4 + e;
              pv = in_span(qrow, key_rows) ? pv : 0.f;
            }
            pt[mq][r] = pv;
            dst[mq][r] = pv * dst[mq][r];  // dS = P (dP - D)
          }
        }
      // dV^T[d x keys] += dO^T[d x q] P[q x keys];  dK^T += Q^T dS
#pragma unroll
      for (int s = 0; s < C::BMB / KS; ++s) {
        const typename M::Frag pf = pack_frag<T>(pt, s);
        const typename M::Frag sf = pack_frag<T>(dst, s);
#pragma unroll
        for (int md = 0; md < D / 32; ++md) {
          dvt[md] = M::mma(frag_col<T, C::BMB>(fa, dOs, md, s), pf, dvt[md]);
          dkt[md] = M::mma(frag_col<T, C::BMB>(fa, Qs, md, s), sf, dkt[md]);
        }
      }
    };
    auto step = [&](int it, int qt, auto full_tag) __device__ {
      constexpr bool FULL = decltype(full_tag)::value;
      const int buf = it % NB;
      if constexpr (DkvCfg<T, D>::PER_CU == 2) {
        if (young && (it % 3 != 0)) __builtin_amdgcn_s_setprio(1); else __builtin_amdgcn_s_setprio(0);
      }
      // bf16: tile it+2 goes to the buffer read in the previous step; fp32: tile it+1.
      const bool more = it + NB - 1 < n_it;
      if (more) stage(it + NB - 1, (it + NB - 1) % NB);
      const int qbase = qt * TP;  // first query position of the tile
      if constexpr (FULL) {
        body(buf, qbase, full_tag);
      } else {
        const int qlast = min(qbase + TP, nq) - 1;
        if (wave_keys && qbase < wqhi && qlast >= wqlo) body(buf, qbase, full_tag);
      }
      if constexpr (NB == 3) {
        // Tile it+1 must have landed; tile it+2's DMAs (this wavefront's last
        // kStageVm vector-memory instructions, plus the lse / -D row on waves 0 and
        // 1) may still fly.
        if (more) {
          if (w < 2)
            wait_vmcnt<kStageVm + 1>();
          else
            wait_vmcnt<kStageVm>();
        } else {
          wait_vmcnt<0>();
        }
      } else {
        if (more) commit((it + 1) % NB);
      }
      __syncthreads();
    };
    // Query tiles [qf_lo, qf_hi) are fully visible to all 32 keys of this wavefront:
    // past the diagonal, before the window's right edge, inside the sequence.
    const int qt_end = qt_begin + nqt;
    int qf_lo = qt_begin, qf_hi = qt_begin;
    if (kw + 32 <= nk) {
      const int lo_q = f.causal ? kw + 31 - off : 0;                      // first row seeing all 32 keys
      const int hi_q = f.window > 0 ? min(kw - off + f.window, nq) : nq;  // rows below this see them too
      qf_lo = clampi(lo_q > 0 ? (lo_q + TP - 1) / TP : 0, qt_begin, qt_end);
      qf_hi = clampi(hi_q > 0 ? hi_q / TP : 0, qf_lo, qt_end);
    }
    int it = 0;
    for (int hd = 0; hd < (PKH ? 1 : hps); ++hd) {
      if constexpr (DOWN) {
        int qt = qt_end - 1;
        for (; qt >= qf_hi; --qt, ++it) step(it, qt, std::false_type{});
        for (; qt >= qf_lo; --qt, ++it) step(it, qt, std::true_type{});
        for (; qt >= qt_begin; --qt, ++it) step(it, qt, std::false_type{});
      } else {
        int qt = qt_begin;
        for (; qt < qf_lo; ++qt, ++it) step(it, qt, std::false_type{});
        for (; qt < qf_hi; ++qt, ++it) step(it, qt, std::true_type{});
        for (; qt < qt_end; ++qt, ++it) step(it, qt, std::false_type{});
      }
    }

    // Lane owns key kj; register r of tile md holds d = 32 md + crow(r, h).
    if (kok) {
      const size_t o = (size_t)(sk.start + kj) * kv_row + g * D;
#pragma unroll
      for (int md = 0; md < D / 32; ++md)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = 32 * md + crow(4 * r4, h);
          const f32x16& tk = dkt[md];
          const f32x16& tv = dvt[md];
          if (a.splits == 1) {
            T* dk = static_cast<T*>(a.dk) + o + d0;
            T* dv = static_cast<T*>(a.dv) + o + d0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              dk[e] = from_f32<T>(tk[4 * r4 + e] * f.scale);
              dv[e] = from_f32<T>(tv[4 * r4 + e]);
            }
          } else {
            const size_t so = (size_t)split * f.total_k * kv_row + o + d0;
            *reinterpret_cast<f32x4*>(a.dk_part + so) = f32x4{tk[4 * r4], tk[4 * r4 + 1], tk[4 * r4 + 2], tk[4 * r4 + 3]};
            *reinterpret_cast<f32x4*>(a.dv_part + so) = f32x4{tv[4 * r4], tv[4 * r4 + 1], tv[4 * r4 + 2], tv[4 * r4 + 3]};
          }
        }
    }
  }
}

// ----------------------------------------------------------------------------- 3. finish
template <typename T>
__global__ __launch_bounds__(256) void bwd_finish_kernel(BwdArgs a) {
  const int D = a.f.d;
  const FwdArgs& f = a.f;
  if ((int)blockIdx.x < f.hq) {
    // dS_h of head blockIdx.x: the preprocess partials, summed in a fixed order
    // (strided per thread, then a fixed butterfly and the four wavefronts in order).
    const float* part = a.dsink_part + (size_t)blockIdx.x * a.pre_blocks;
    // Eight strides' loads are issued before their adds (0 past the end: acc is never
    // -0, so adding +0 leaves it bitwise unchanged and the sum is that of the plain
    // strided loop).
    float acc = 0.f;
    for (int j0 = threadIdx.x; j0 < a.pre_blocks; j0 += 8 * blockDim.x) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u * (int)blockDim.x;
        v[u] = j < a.pre_blocks ? part[j] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += v[u];
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) a.dsinks[blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
  }
  if (a.splits > 1) {
    const size_t n4 = (size_t)f.total_k * f.hkv * D / 4;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x) {
      f32x4 sk = reinterpret_cast<const f32x4*>(a.dk_part)[i];
      f32x4 sv = reinterpret_cast<const f32x4*>(a.dv_part)[i];
      for (int s = 1; s < a.splits; ++s) {
        sk += reinterpret_cast<const f32x4*>(a.dk_part)[i + s * n4];
        sv += reinterpret_cast<const f32x4*>(a.dv_part)[i + s * n4];
      }
      T* dk = static_cast<T*>(a.dk) + 4 * i;
      T* dv = static_cast<T*>(a.dv) + 4 * i;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dk[e] = from_f32<T>(sk[e] * f.scale);
        dv[e] = from_f32<T>(sv[e]);
      }
    }
  }
}

// ----------------------------------------------------------------------------- launchers
template <typename T, int D>
static void launch_bwd_dq_t(const BwdArgs& a, hipStream_t stream) {
  const FwdArgs& f = a.f;
  const int tiles = dq_tiles(f.hq, f.hkv, f.num_seqs, f.max_q, f.window);
  if (dq_head_packed(f.hq, f.hkv, f.num_seqs, f.max_q, f.window))
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, true>), dim3(f.hkv, tiles, f.num_seqs), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, false>), dim3(f.hq * f.num_seqs, tiles), dim3(256), 0, stream, a);
}

hipError_t launch_bwd_dq(const BwdArgs& a, int fp32, hipStream_t stream) {
  if (a.f.max_q == 0) return hipSuccess;
  if (a.f.d == 128) {
    if (fp32)
      launch_bwd_dq_t<float, 128>(a, stream);
    else
      launch_bwd_dq_t<bf16, 128>(a, stream);
  } else {
    if (fp32)
      launch_bwd_dq_t<float, 64>(a, stream);
    else
      launch_bwd_dq_t<bf16, 64>(a, stream);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, int fp32, hipStream_t stream) {
  auto launch = [&](auto kernel, int bnb, int threads) {
    const int ktiles = (a.f.max_k + bnb - 1) / bnb;
    if (ktiles == 0) return;
    const int nfold = (ktiles + 1) / 2;
    // Several sequences: sequence-major rows (measured on the ragged 8-sequence batch, 49.8k
    // rows: window-128 layer 537 against 710 us, full causal layer 7.23 against 8.35 ms).
    dim3 grid = a.f.num_seqs > 1 && (long long)a.f.num_seqs * nfold <= 65535
                    ? dim3(a.f.hkv * a.splits, a.f.num_seqs * nfold)
                    : dim3(a.f.hkv * a.splits * a.f.num_seqs, nfold);
    hipLaunchKernelGGL(kernel, grid, dim3(threads), 0, stream, a);
  };
  if (!fp32 && dkdv_head_packed(a.f.hq, a.f.hkv, a.f.window, a.splits)) {
    if (a.f.d == 128)
      launch(bwd_dkdv_kernel<bf16, 128, true>, DkvCfg<bf16, 128>::BNB, DkvCfg<bf16, 128>::THREADS);
    else
      launch(bwd_dkdv_kernel<bf16, 64, true>, DkvCfg<bf16, 64>::BNB, DkvCfg<bf16, 64>::THREADS);
  } else if (a.f.d == 128) {
    if (fp32)
      launch(bwd_dkdv_kernel<float, 128, false>, DkvCfg<float, 128>::BNB, DkvCfg<float, 128>::THREADS);
    else
      launch(bwd_dkdv_kernel<bf16, 128, false>, DkvCfg<bf16, 128>::BNB, DkvCfg<bf16, 128>::THREADS);
  } else {
    if (fp32)
      launch(bwd_dkdv_kernel<float, 64, false>, DkvCfg<float, 64>::BNB, DkvCfg<float, 64>::THREADS);
    else
      launch(bwd_dkdv_kernel<bf16, 64, false>, DkvCfg<bf16, 64>::BNB, DkvCfg<bf16, 64>::THREADS);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_finish(const BwdArgs& a, int fp32, hipStream_t stream) {
  size_t blocks = 1;
  if (a.splits > 1) {
    const size_t n4 = (size_t)a.f.total_k * a.f.hkv * a.f.d / 4;
    blocks = (n4 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks == 0) blocks = 1;
  }
  if (blocks < (size_t)a.f.hq) blocks = a.f.hq;  // one block per head for dS_h
  if (fp32)
    hipLaunchKernelGGL(bwd_finish_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_finish_kernel<bf16>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn_sink
