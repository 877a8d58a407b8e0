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
//   * K (row-major) and V^T (transposed while staging) tiles of 64 keys go through
//     LDS, double-buffered with register prefetch; padded strides keep the MFMA
//     operand reads free of bank conflicts.
//   * Online softmax in the exp2 domain.  The running max starts at the sink logit
//     S_h*log2(e) (not at -inf), so every exponent stays <= 0; the sink's own mass
//     exp2(S_h*log2e - m) is added once at the end.  S_h = -inf is standard
//     attention: the guarded max m_use avoids exp2(-inf - -inf).
//   * O^T = V^T P^T reuses the S^T accumulator registers as the B operand (P
//     rounded to the element type), so P never leaves registers.
//   * Tiles outside the causal / sliding-window band are never visited; the mask
//     is evaluated only on tiles that straddle a band edge or the sequence end.
//   * Longest query tiles are dispatched first (causal load balance), and the
//     query heads that share a kv head are placed on one XCD so their K/V tiles
//     hit the same L2.
#include "common.h"
#include "kernels.h"

namespace attn_sink {

template <typename T>
struct FwdCfg {
  static constexpr int BM = 128;           // query rows per workgroup
  static constexpr int BN = 64;            // keys per tile
  static constexpr int THREADS = 256;      // 4 wavefronts x 32 rows
  static constexpr int VEC = 16 / sizeof(T);            // elements per 16-byte chunk
  static constexpr int CPR = kD / VEC;                   // chunks per row
  static constexpr int KSTR = sizeof(T) == 2 ? 72 : 65;  // K tile row stride (elements)
  static constexpr int VSTR = sizeof(T) == 2 ? 68 : 65;  // V^T tile row stride (elements)
  static constexpr int K_ELEMS = BN * KSTR;
  static constexpr int V_ELEMS = kD * VSTR;
  static constexpr int K_CHUNKS = BN * CPR / THREADS;    // K chunks per thread
  static constexpr int V_ROWS = sizeof(T) == 2 ? 2 : 1;  // key rows per V^T task
  static constexpr int V_TASKS = (BN / V_ROWS) * CPR / THREADS;
};

__device__ inline bool visible(int i, int j, int off, int nk, int causal, int window) {
  return j < nk && (!causal || j <= i + off) && (window <= 0 || j > i + off - window);
}

// Map a flat workgroup index over (head, seq) so that the Hq/Hkv heads of one kv
// head land on one XCD (workgroups are dealt to the 8 XCDs round-robin).
__device__ inline int xcd_remap(int x, int n) {
  if (n % 8 != 0) return x;
  return (x % 8) * (n / 8) + x / 8;
}

template <typename T>
__global__ __launch_bounds__(256) void fwd_kernel(FwdArgs p) {
  using C = FwdCfg<T>;
  using M = Mfma<T>;
  constexpr int E = M::E, KS = M::KS;
  __shared__ __attribute__((aligned(16))) T smem[2 * (C::K_ELEMS + C::V_ELEMS)];

  const int n_hs = p.hq * p.num_seqs;
  const int hs = xcd_remap(blockIdx.x, n_hs);
  const int head = hs % p.hq;
  const int b = hs / p.hq;
  const int tile = gridDim.y - 1 - blockIdx.y;  // longest causal tiles first
  const int g = head / (p.hq / p.hkv);

  const SeqBounds sq = seq_bounds(p.cu_q, b, p.total_q);
  const SeqBounds sk = seq_bounds(p.cu_k, b, p.total_k);
  const int nq = sq.len, nk = sk.len, off = nk - nq;
  const int qs = tile * C::BM;
  if (qs >= nq) return;
  const int qe = min(qs + C::BM, nq);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, c = lane & 31;

  // Key range of the workgroup and of this wavefront.
  int khi = p.causal ? clampi(qe - 1 + off + 1, 0, nk) : nk;
  int klo = p.window > 0 ? clampi(qs + off - p.window + 1, 0, nk) : 0;
  const int qw = qs + 32 * w;
  const int qw_end = min(qw + 32, nq);
  const bool wave_rows = qw < nq;
  int whi = p.causal ? clampi(qw_end - 1 + off + 1, 0, nk) : nk;
  int wlo = p.window > 0 ? clampi(qw + off - p.window + 1, 0, nk) : 0;
  if (!wave_rows) { whi = 0; wlo = 0; }

  const T* __restrict__ qp = static_cast<const T*>(p.q);
  const T* __restrict__ kp = static_cast<const T*>(p.k);
  const T* __restrict__ vp = static_cast<const T*>(p.v);
  const size_t kv_row = (size_t)p.hkv * kD;

  // Q fragments (B operand of S^T = K Q^T): lane owns query qw + c, d = KS*s + E*h + e.
  const int qi = qw + c;
  typename M::Frag qf[kD / KS];
  {
    const bool ok = qi < nq;
    const T* src = qp + ((size_t)(sq.start + (ok ? qi : 0)) * p.hq + head) * kD;
#pragma unroll
    for (int s = 0; s < kD / KS; ++s) {
      if constexpr (E == 8) {
        uint4 v = ok ? ld16(src + KS * s + E * h) : make_uint4(0, 0, 0, 0);
        qf[s] = *reinterpret_cast<bf16x8*>(&v);
      } else {
        qf[s] = ok ? src[KS * s + h] : 0.f;
      }
    }
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

  // ---- staging: global -> registers -> LDS
  uint4 kreg[C::K_CHUNKS];
  uint4 vreg[C::V_TASKS][C::V_ROWS];
  auto load_regs = [&](int kt) {
    const int kbase = kt * C::BN;
#pragma unroll
    for (int i = 0; i < C::K_CHUNKS; ++i) {
      const int ch = tid + C::THREADS * i;
      const int row = ch / C::CPR, col = ch % C::CPR;
      const int key = kbase + row;
      kreg[i] = key < nk ? ld16(kp + (size_t)(sk.start + key) * kv_row + g * kD + col * C::VEC)
                         : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::V_TASKS; ++i) {
      const int task = tid + C::THREADS * i;
      const int col = task % C::CPR, kr = task / C::CPR;
#pragma unroll
      for (int rr = 0; rr < C::V_ROWS; ++rr) {
        const int key = kbase + kr * C::V_ROWS + rr;
        vreg[i][rr] = key < nk ? ld16(vp + (size_t)(sk.start + key) * kv_row + g * kD + col * C::VEC)
                               : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_lds = [&](int buf) {
    T* Ks = smem + buf * (C::K_ELEMS + C::V_ELEMS);
    T* Vt = Ks + C::K_ELEMS;
#pragma unroll
    for (int i = 0; i < C::K_CHUNKS; ++i) {
      const int ch = tid + C::THREADS * i;
      const int row = ch / C::CPR, col = ch % C::CPR;
      T* dst = Ks + row * C::KSTR + col * C::VEC;
      if constexpr (sizeof(T) == 2) {
        st16(dst, kreg[i]);
      } else {
        const float* f = reinterpret_cast<const float*>(&kreg[i]);
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e] = f[e];
      }
    }
#pragma unroll
    for (int i = 0; i < C::V_TASKS; ++i) {
      const int task = tid + C::THREADS * i;
      const int col = task % C::CPR, kr = task / C::CPR;
      if constexpr (sizeof(T) == 2) {
        const bf16* a = reinterpret_cast<const bf16*>(&vreg[i][0]);
        const bf16* bb = reinterpret_cast<const bf16*>(&vreg[i][1]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bf16x2 pr = {a[e], bb[e]};
          *reinterpret_cast<bf16x2*>(Vt + (col * 8 + e) * C::VSTR + 2 * kr) = pr;
        }
      } else {
        const float* f = reinterpret_cast<const float*>(&vreg[i][0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) Vt[(col * 4 + e) * C::VSTR + kr] = f[e];
      }
    }
  };

  if (kt_begin < kt_end) {
    load_regs(kt_begin);
    store_lds(0);
  }
  __syncthreads();

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int buf = (kt - kt_begin) & 1;
    if (kt + 1 < kt_end) load_regs(kt + 1);
    const int kbase = kt * C::BN;
    if (kbase < whi && kbase + C::BN > wlo) {
      const T* Ks = smem + buf * (C::K_ELEMS + C::V_ELEMS);
      const T* Vt = Ks + C::K_ELEMS;
      // S^T tile [64 keys x 32 queries] as two 32x32 tiles.
      f32x16 sacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[mt][r] = 0.f;
#pragma unroll
        for (int s = 0; s < kD / KS; ++s)
          sacc[mt] = M::mma(lds_frag<T>(Ks + (32 * mt + c) * C::KSTR + KS * s + E * h), qf[s], sacc[mt]);
      }
      // Mask only where the tile straddles the band edge or the sequence end.
      const bool full = kbase + C::BN <= nk && (!p.causal || kbase + C::BN - 1 <= qw + off) &&
                        (p.window <= 0 || kbase > qw_end - 1 + off - p.window);
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = sacc[mt][r] * sl2;
          if (!full && !visible(qi, kbase + 32 * mt + crow(r, h), off, nk, p.causal, p.window)) x = -INFINITY;
          sacc[mt][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float psum = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = fast_exp2(sacc[mt][r] - m_use);
          sacc[mt][r] = pr;
          psum += pr;
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;
      // O^T[d x q] += V^T[d x keys] . P^T[keys x q]
#pragma unroll
      for (int s = 0; s < C::BN / KS; ++s) {
        const typename M::Frag pf = pack_frag<T>(sacc, s);
#pragma unroll
        for (int md = 0; md < 2; ++md) {
          const T* row = Vt + (32 * md + c) * C::VSTR;
          oacc[md] = M::mma(lds_frag_split<T>(row + kc(E * s, h), row + kc(E * s + (E == 8 ? 4 : 0), h)), pf,
                            oacc[md]);
        }
      }
    }
    if (kt + 1 < kt_end) store_lds(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: add the sink's mass once, normalise, write O and LSE.
  const float m_use = m_run == -INFINITY ? 0.f : m_run;
  float l_tot = l_run + __shfl_xor(l_run, 32);
  if (sink2 > -INFINITY) l_tot += fast_exp2(sink2 - m_use);
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
