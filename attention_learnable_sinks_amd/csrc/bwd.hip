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
// Three kernels on one stream:
//   1. bwd_pre:    D_i, per-block partial sums of -P_sink_i D_i (reduced later in a
//                  fixed order, so dS_h is bitwise reproducible), and zeroing of the
//                  fp32 accumulators.
//   2. bwd_dkdv:   one workgroup per (128 keys, query head).  Wavefront w owns keys
//                  32w..32w+31 and keeps K, V in registers and dK^T, dV^T in fp32
//                  accumulators across the query band.  Per 64-query tile, Q and dO
//                  are staged in LDS row-major and transposed; S = Q K^T and
//                  dP = dO V^T put the key on the lane, so P and dS feed dV^T += dO^T P
//                  and dK^T += Q^T dS straight from registers.  dS goes through LDS
//                  once more for dQ = dS K, which is added to an fp32 buffer with
//                  hardware float atomics.  dK/dV of the Hq/Hkv query heads that share
//                  a kv head are summed with float atomics at the end.
//   3. bwd_finish: scale and round dq/dk/dv to the element type; sum dS_h partials.
#include "common.h"
#include "kernels.h"

namespace attn_sink {

constexpr int kPreRows = 64;  // rows per bwd_pre workgroup

__device__ inline bool visible(int i, int j, int off, int nk, int causal, int window) {
  return j < nk && (!causal || j <= i + off) && (window <= 0 || j > i + off - window);
}

__device__ inline int xcd_remap(int x, int n) {
  if (n % 8 != 0) return x;
  return (x % 8) * (n / 8) + x / 8;
}

// ----------------------------------------------------------------------------- 1. preprocess
template <typename T>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
  const FwdArgs& f = a.f;
  const int head = blockIdx.y;
  const int tid = threadIdx.x;
  const int row = blockIdx.x * kPreRows + tid / 4;
  const int part = tid % 4;  // 16 of the 64 columns
  float contrib = 0.f;
  if (head < f.hq && row < f.total_q) {
    const size_t base = ((size_t)row * f.hq + head) * kD + part * 16;
    const T* o = static_cast<const T*>(f.o) + base;
    const T* d = static_cast<const T*>(a.dout) + base;
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc += to_f32(o[e]) * to_f32(d[e]);
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) *reinterpret_cast<f32x4*>(a.dq_acc + base + 4 * e) = z;
    if (part == 0) {
      a.delta[(size_t)head * f.total_q + row] = acc;
      const float lse = f.lse[(size_t)head * f.total_q + row];
      const float sink = f.sinks[head];
      const float ps = (lse > -INFINITY && sink > -INFINITY) ? fast_exp2((sink - lse) * kLog2e) : 0.f;
      contrib = -ps * acc;
    }
  }
  if (head < f.hkv && row < f.total_k) {
    const size_t base = ((size_t)row * f.hkv + head) * kD + part * 16;
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      *reinterpret_cast<f32x4*>(a.dk_acc + base + 4 * e) = z;
      *reinterpret_cast<f32x4*>(a.dv_acc + base + 4 * e) = z;
    }
  }
  // Fixed-order block reduction of the sink-gradient contributions.
  __shared__ float red[4];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) contrib += __shfl_xor(contrib, m);
  if ((tid & 63) == 0) red[tid >> 6] = contrib;
  __syncthreads();
  if (tid == 0 && head < f.hq) a.dsink_part[(size_t)head * a.pre_blocks + blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

// ----------------------------------------------------------------------------- 2. dK, dV (+ dQ atomics)
template <typename T>
struct BwdCfg {
  static constexpr int BMB = 64;    // queries per tile
  static constexpr int BNB = 128;   // keys per workgroup (4 wavefronts x 32)
  static constexpr int THREADS = 256;
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int CPR = kD / VEC;
  static constexpr int QSTR = sizeof(T) == 2 ? 72 : 65;    // [64 q][64 d]
  static constexpr int TSTR = sizeof(T) == 2 ? 68 : 65;    // [64 d][64 q]
  static constexpr int SSTR = sizeof(T) == 2 ? 136 : 129;  // [64 q][128 k] and [64 d][128 k]
  static constexpr int Q_ELEMS = BMB * QSTR;
  static constexpr int T_ELEMS = kD * TSTR;
  static constexpr int S_ELEMS = BMB * SSTR;
  static constexpr int KT_ELEMS = kD * SSTR;
  static constexpr int ROWS = sizeof(T) == 2 ? 2 : 1;                 // rows per staging task
  static constexpr int TASKS = (BMB / ROWS) * CPR / THREADS;          // per tensor, per thread
  static constexpr int KT_TASKS = (BNB / ROWS) * CPR / THREADS;
};

template <typename T>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(BwdArgs a) {
  using C = BwdCfg<T>;
  using M = Mfma<T>;
  constexpr int E = M::E, KS = M::KS;
  const FwdArgs& f = a.f;
  __shared__ __attribute__((aligned(16))) T smem[2 * C::Q_ELEMS + 2 * C::T_ELEMS + C::S_ELEMS + C::KT_ELEMS];
  __shared__ __attribute__((aligned(16))) float lse2_s[C::BMB];
  __shared__ __attribute__((aligned(16))) float dd_s[C::BMB];
  T* Qs = smem;
  T* dOs = Qs + C::Q_ELEMS;
  T* QsT = dOs + C::Q_ELEMS;
  T* dOsT = QsT + C::T_ELEMS;
  T* dSs = dOsT + C::T_ELEMS;
  T* KsT = dSs + C::S_ELEMS;

  const int n_hs = f.hq * f.num_seqs;
  const int hs = xcd_remap(blockIdx.x, n_hs);
  const int head = hs % f.hq;
  const int b = hs / f.hq;
  const int ktile = blockIdx.y;  // low key tiles see the most queries under a causal mask
  const int g = head / (f.hq / f.hkv);

  const SeqBounds sq = seq_bounds(f.cu_q, b, f.total_q);
  const SeqBounds sk = seq_bounds(f.cu_k, b, f.total_k);
  const int nq = sq.len, nk = sk.len, off = nk - nq;
  const int kbase = ktile * C::BNB;
  if (kbase >= nk) return;
  const int kend = min(kbase + C::BNB, nk);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, c = lane & 31;

  // Query band of the workgroup and of this wavefront's 32 keys.
  const int qlo = f.causal ? clampi(kbase - off, 0, nq) : 0;
  const int qhi = f.window > 0 ? clampi(kend - 1 - off + f.window, 0, nq) : nq;
  const int kw = kbase + 32 * w;
  const int kw_end = min(kw + 32, nk);
  const bool wave_keys = kw < nk;
  const int wqlo = f.causal ? clampi(kw - off, 0, nq) : 0;
  const int wqhi = f.window > 0 ? clampi(kw_end - 1 - off + f.window, 0, nq) : nq;

  const T* __restrict__ qp = static_cast<const T*>(f.q);
  const T* __restrict__ kp = static_cast<const T*>(f.k);
  const T* __restrict__ vp = static_cast<const T*>(f.v);
  const T* __restrict__ dop = static_cast<const T*>(a.dout);
  const size_t kv_row = (size_t)f.hkv * kD;
  const size_t q_row = (size_t)f.hq * kD;

  // K and V fragments (B operands of S = Q K^T and dP = dO V^T): lane owns key kw + c.
  const int kj = kw + c;
  typename M::Frag kf[kD / KS], vf[kD / KS];
  {
    const bool ok = kj < nk;
    const size_t off_kv = (size_t)(sk.start + (ok ? kj : 0)) * kv_row + g * kD;
#pragma unroll
    for (int s = 0; s < kD / KS; ++s) {
      if constexpr (E == 8) {
        uint4 k4 = ok ? ld16(kp + off_kv + KS * s + E * h) : make_uint4(0, 0, 0, 0);
        uint4 v4 = ok ? ld16(vp + off_kv + KS * s + E * h) : make_uint4(0, 0, 0, 0);
        kf[s] = *reinterpret_cast<bf16x8*>(&k4);
        vf[s] = *reinterpret_cast<bf16x8*>(&v4);
      } else {
        kf[s] = ok ? kp[off_kv + KS * s + h] : 0.f;
        vf[s] = ok ? vp[off_kv + KS * s + h] : 0.f;
      }
    }
  }

  // K^T of the workgroup's 128 keys for dQ = dS K (B operand: lane owns a column d).
#pragma unroll
  for (int i = 0; i < C::KT_TASKS; ++i) {
    const int task = tid + C::THREADS * i;
    const int col = task % C::CPR, kr = task / C::CPR;
    if constexpr (sizeof(T) == 2) {
      uint4 r2[2];
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int key = kbase + 2 * kr + rr;
        r2[rr] = key < nk ? ld16(kp + (size_t)(sk.start + key) * kv_row + g * kD + col * 8) : make_uint4(0, 0, 0, 0);
      }
      const bf16* x0 = reinterpret_cast<const bf16*>(&r2[0]);
      const bf16* x1 = reinterpret_cast<const bf16*>(&r2[1]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16x2 pr = {x0[e], x1[e]};
        *reinterpret_cast<bf16x2*>(KsT + (col * 8 + e) * C::SSTR + 2 * kr) = pr;
      }
    } else {
      const int key = kbase + kr;
      uint4 r = key < nk ? ld16(kp + (size_t)(sk.start + key) * kv_row + g * kD + col * 4) : make_uint4(0, 0, 0, 0);
      const float* x = reinterpret_cast<const float*>(&r);
#pragma unroll
      for (int e = 0; e < 4; ++e) KsT[(col * 4 + e) * C::SSTR + kr] = x[e];
    }
  }

  f32x16 dkt[2], dvt[2];  // [64 d x 32 keys] each, two 32x32 tiles
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dkt[t][r] = 0.f;
      dvt[t][r] = 0.f;
    }

  const float sl2 = f.scale * kLog2e;
  const int qt_begin = qlo / C::BMB;
  const int qt_end = qhi > qlo ? (qhi + C::BMB - 1) / C::BMB : qt_begin;

  // Staging registers for one Q tile and one dO tile.
  uint4 qreg[C::TASKS][C::ROWS], dreg[C::TASKS][C::ROWS];
  float lse_r = 0.f, dd_r = 0.f;
  auto load_regs = [&](int qt) {
    const int qbase = qt * C::BMB;
#pragma unroll
    for (int i = 0; i < C::TASKS; ++i) {
      const int task = tid + C::THREADS * i;
      const int col = task % C::CPR, rr0 = task / C::CPR;
#pragma unroll
      for (int rr = 0; rr < C::ROWS; ++rr) {
        const int qi = qbase + rr0 * C::ROWS + rr;
        const size_t o = (size_t)(sq.start + qi) * q_row + head * kD + col * C::VEC;
        qreg[i][rr] = qi < nq ? ld16(qp + o) : make_uint4(0, 0, 0, 0);
        dreg[i][rr] = qi < nq ? ld16(dop + o) : make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < C::BMB) {
      const int qi = qbase + tid;
      lse_r = qi < nq ? f.lse[(size_t)head * f.total_q + sq.start + qi] * kLog2e : 0.f;
      dd_r = qi < nq ? a.delta[(size_t)head * f.total_q + sq.start + qi] : 0.f;
    }
  };
  auto store_one = [&](T* rowmaj, T* trans, const uint4 (&reg)[C::TASKS][C::ROWS]) {
#pragma unroll
    for (int i = 0; i < C::TASKS; ++i) {
      const int task = tid + C::THREADS * i;
      const int col = task % C::CPR, rr0 = task / C::CPR;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) st16(rowmaj + (2 * rr0 + rr) * C::QSTR + col * 8, reg[i][rr]);
        const bf16* x0 = reinterpret_cast<const bf16*>(&reg[i][0]);
        const bf16* x1 = reinterpret_cast<const bf16*>(&reg[i][1]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bf16x2 pr = {x0[e], x1[e]};
          *reinterpret_cast<bf16x2*>(trans + (col * 8 + e) * C::TSTR + 2 * rr0) = pr;
        }
      } else {
        const float* x = reinterpret_cast<const float*>(&reg[i][0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          rowmaj[rr0 * C::QSTR + col * 4 + e] = x[e];
          trans[(col * 4 + e) * C::TSTR + rr0] = x[e];
        }
      }
    }
  };

  if (qt_begin < qt_end) load_regs(qt_begin);
  for (int qt = qt_begin; qt < qt_end; ++qt) {
    store_one(Qs, QsT, qreg);
    store_one(dOs, dOsT, dreg);
    if (tid < C::BMB) {
      lse2_s[tid] = lse_r;
      dd_s[tid] = dd_r;
    }
    __syncthreads();  // (A) tile staged; the previous tile's dQ reads of dSs are done
    if (qt + 1 < qt_end) load_regs(qt + 1);

    const int qbase = qt * C::BMB;
    const int qlast = min(qbase + C::BMB, nq) - 1;
    const bool active = wave_keys && qbase < wqhi && qlast >= wqlo;
    f32x16 pt[2], dst[2];  // P and dS, [32 q x 32 keys] x 2, key on the lane
    if (active) {
      f32x16 sacc[2], dpacc[2];
#pragma unroll
      for (int mq = 0; mq < 2; ++mq) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[mq][r] = 0.f;
          dpacc[mq][r] = 0.f;
        }
#pragma unroll
        for (int s = 0; s < kD / KS; ++s) {
          sacc[mq] = M::mma(lds_frag<T>(Qs + (32 * mq + c) * C::QSTR + KS * s + E * h), kf[s], sacc[mq]);
          dpacc[mq] = M::mma(lds_frag<T>(dOs + (32 * mq + c) * C::QSTR + KS * s + E * h), vf[s], dpacc[mq]);
        }
      }
      const bool full = qbase + C::BMB <= nq && kw_end == kw + 32 &&
                        (!f.causal || kw + 31 <= qbase + off) &&
                        (f.window <= 0 || kw > qlast + off - f.window);
#pragma unroll
      for (int mq = 0; mq < 2; ++mq)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int ql = 32 * mq + crow(4 * r4, h);  // 4 consecutive query rows
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2_s + ql);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(dd_s + ql);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * r4 + e;
            float pv = fast_exp2(sacc[mq][r] * sl2 - l4[e]);
            if (!full && !(qbase + ql + e < nq && visible(qbase + ql + e, kj, off, nk, f.causal, f.window))) pv = 0.f;
            pt[mq][r] = pv;
            dst[mq][r] = pv * (dpacc[mq][r] - d4[e]);
          }
        }
      // dV^T[d x keys] += dO^T[d x q] P[q x keys];  dK^T += Q^T dS
#pragma unroll
      for (int s = 0; s < C::BMB / KS; ++s) {
        const typename M::Frag pf = pack_frag<T>(pt, s);
        const typename M::Frag sf = pack_frag<T>(dst, s);
#pragma unroll
        for (int md = 0; md < 2; ++md) {
          const T* rd = dOsT + (32 * md + c) * C::TSTR;
          const T* rq = QsT + (32 * md + c) * C::TSTR;
          const int k0 = kc(E * s, h), k1 = kc(E * s + (E == 8 ? 4 : 0), h);
          dvt[md] = M::mma(lds_frag_split<T>(rd + k0, rd + k1), pf, dvt[md]);
          dkt[md] = M::mma(lds_frag_split<T>(rq + k0, rq + k1), sf, dkt[md]);
        }
      }
    } else {
#pragma unroll
      for (int mq = 0; mq < 2; ++mq)
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[mq][r] = 0.f;
    }
    // dS -> LDS as [q][key] for dQ = dS K.
#pragma unroll
    for (int mq = 0; mq < 2; ++mq)
#pragma unroll
      for (int r = 0; r < 16; ++r) dSs[(32 * mq + crow(r, h)) * C::SSTR + 32 * w + c] = from_f32<T>(dst[mq][r]);
    __syncthreads();  // (B) dSs complete; all reads of Qs/dOs for this tile are done

    // dQ tile [32 q x 32 d] per wavefront over the 128 keys, accumulated with atomics.
    {
      const int mq = w >> 1, md = w & 1;
      f32x16 dqa;
#pragma unroll
      for (int r = 0; r < 16; ++r) dqa[r] = 0.f;
#pragma unroll
      for (int s = 0; s < C::BNB / KS; ++s)
        dqa = M::mma(lds_frag<T>(dSs + (32 * mq + c) * C::SSTR + KS * s + E * h),
                     lds_frag<T>(KsT + (32 * md + c) * C::SSTR + KS * s + E * h), dqa);
      float* dq_base = a.dq_acc + (size_t)head * kD + 32 * md + c;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = qbase + 32 * mq + crow(r, h);
        if (qi < nq) atomicAdd(dq_base + (size_t)(sq.start + qi) * q_row, dqa[r]);
      }
    }
  }

  // dK^T / dV^T: lane owns key kj; register r of tile md holds d = 32 md + crow(r, h).
  if (kj < nk && qt_begin < qt_end) {
    float* dkb = a.dk_acc + (size_t)(sk.start + kj) * kv_row + g * kD;
    float* dvb = a.dv_acc + (size_t)(sk.start + kj) * kv_row + g * kD;
#pragma unroll
    for (int md = 0; md < 2; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        atomicAdd(dkb + 32 * md + crow(r, h), dkt[md][r]);
        atomicAdd(dvb + 32 * md + crow(r, h), dvt[md][r]);
      }
  }
}

// ----------------------------------------------------------------------------- 3. finish
template <typename T>
__global__ __launch_bounds__(256) void bwd_finish_kernel(BwdArgs a) {
  const FwdArgs& f = a.f;
  const size_t nq4 = (size_t)f.total_q * f.hq * kD / 4;
  const size_t nk4 = (size_t)f.total_k * f.hkv * kD / 4;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nq4) {
    const f32x4 x = reinterpret_cast<const f32x4*>(a.dq_acc)[i];
    T* d = static_cast<T*>(a.dq) + 4 * i;
#pragma unroll
    for (int e = 0; e < 4; ++e) d[e] = from_f32<T>(x[e] * f.scale);
  }
  if (i < nk4) {
    const f32x4 x = reinterpret_cast<const f32x4*>(a.dk_acc)[i];
    const f32x4 y = reinterpret_cast<const f32x4*>(a.dv_acc)[i];
    T* dk = static_cast<T*>(a.dk) + 4 * i;
    T* dv = static_cast<T*>(a.dv) + 4 * i;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dk[e] = from_f32<T>(x[e] * f.scale);
      dv[e] = from_f32<T>(y[e]);
    }
  }
  if (blockIdx.x == 0) {
    for (int hh = threadIdx.x; hh < f.hq; hh += blockDim.x) {
      const float* part = a.dsink_part + (size_t)hh * a.pre_blocks;
      float s = 0.f;
      for (int j = 0; j < a.pre_blocks; ++j) s += part[j];
      a.dsinks[hh] = s;
    }
  }
}

// ----------------------------------------------------------------------------- launchers
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

BwdWorkspace bwd_workspace_layout(int hq, int hkv, int total_q, int total_k) {
  BwdWorkspace w;
  const int rows = total_q > total_k ? total_q : total_k;
  w.pre_blocks = (rows + kPreRows - 1) / kPreRows;
  if (w.pre_blocks == 0) w.pre_blocks = 1;
  size_t o = 0;
  w.dq_acc = o;      o = align256(o + (size_t)total_q * hq * kD * 4);
  w.dk_acc = o;      o = align256(o + (size_t)total_k * hkv * kD * 4);
  w.dv_acc = o;      o = align256(o + (size_t)total_k * hkv * kD * 4);
  w.delta = o;       o = align256(o + (size_t)hq * total_q * 4);
  w.dsink_part = o;  o = align256(o + (size_t)hq * w.pre_blocks * 4);
  w.total = o;
  return w;
}

hipError_t launch_bwd_pre(const BwdArgs& a, int fp32, hipStream_t stream) {
  const int heads = a.f.hq > a.f.hkv ? a.f.hq : a.f.hkv;
  dim3 grid(a.pre_blocks, heads);
  if (fp32)
    hipLaunchKernelGGL(bwd_pre_kernel<float>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_pre_kernel<bf16>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, int fp32, hipStream_t stream) {
  const int ktiles = (a.f.max_k + BwdCfg<bf16>::BNB - 1) / BwdCfg<bf16>::BNB;
  if (ktiles == 0 || a.f.num_seqs == 0) return hipSuccess;
  dim3 grid(a.f.hq * a.f.num_seqs, ktiles);
  if (fp32)
    hipLaunchKernelGGL(bwd_dkdv_kernel<float>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_dkdv_kernel<bf16>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_finish(const BwdArgs& a, int fp32, hipStream_t stream) {
  const size_t nq4 = (size_t)a.f.total_q * a.f.hq * kD / 4;
  const size_t nk4 = (size_t)a.f.total_k * a.f.hkv * kD / 4;
  size_t n = nq4 > nk4 ? nq4 : nk4;
  if (n == 0) n = 1;
  dim3 grid((unsigned)((n + 255) / 256));
  if (fp32)
    hipLaunchKernelGGL(bwd_finish_kernel<float>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_finish_kernel<bf16>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn_sink
