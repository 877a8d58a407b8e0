// Forward of attention with per-head learnable sinks for a few query rows per
// sequence against long key ranges (a decoding step, or a short chunk, against a KV
// cache), on gfx950.
//
// Same function as the forward kernel -- per query row i of head h
//   o_i = sum_j P_ij v_j,  P_ij = exp(s_ij) / (sum_j' exp(s_ij') + exp(S_h)),
//   lse_i = log(sum_j exp(s_ij) + exp(S_h))
// ("Unlocking Agentic RL Training for GPT-OSS", 带汇聚的注意力 and 数学公式: the sink
// joins the normaliser once and never multiplies V) -- organised for the inference
// side, where each sequence contributes one or a few new rows, the key range is
// long, and the kernel only has to stream K and V from HBM once:
//   * The query heads that share a kv head, times the new rows, fill the 32 columns
//     of one MFMA block (column c = query head g*G + c % G, row c / G), so K and V
//     are read once per kv head instead of once per query head.
//   * A workgroup covers one chunk of consecutive key tiles of one sequence for
//     several kv heads at once, one wavefront per kv head.  The wavefronts walk the
//     same key rows in step, so together they read whole contiguous K / V rows
//     (all heads of a token) rather than 128-byte pieces scattered over the cache.
//     Each wavefront stages its tiles in its own LDS region, two deep so the next
//     tile's loads are in flight while it computes on the current one, and keeps
//     an exact online softmax (running max per tile, no sink): no workgroup
//     barrier at all.  Measured on the 64-sequence rollout step this reaches
//     about 0.6 of the HBM peak; a probe that only streams the same tiles in the
//     same pattern reaches 0.78, the rest is per-workgroup start-up and the tail.
//   * Chunks have a fixed number of tiles (1024 keys), so long and short caches
//     cost in proportion to their length, the hardware dispatcher balances the
//     workgroups, and a sequence's result depends on nothing but its own inputs
//     (not on the batch it is decoded in).  A sequence whose visible keys fit in one chunk is finished in
//     place (sink added, normalised, written).  Otherwise each chunk writes a
//     partial (O unnormalised, max m, sum l) and the merge kernel combines the
//     chunks of a row in chunk order, adding the sink's mass exactly once:
//       M = max(S_h, max_c m_c),  L = e^(S_h - M) + sum_c l_c e^(m_c - M),
//       o = sum_c O_c e^(m_c - M) / L,  lse = M + log L      (exp2 domain inside)
//     (folded 16 chunks at a time with a running M, which is the same sum).
//   The results equal the forward kernel's up to rounding order; the summation
//   order is fixed, so they are bitwise repeatable.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace attn_sink {

constexpr int kDecBN = kDecodeKeys;      // keys per tile
constexpr int kDecCols = kDecodeCols;    // (query head, row) columns per kv head
constexpr int kDecWaves = kDecodeWaves;  // wavefronts (kv heads) per workgroup at most

// LDS stages per wavefront.  bf16: two, so the next tile's loads are in flight while
// the wavefront computes on the current one; 4 wavefronts x 2 stages x 8 KB = 64 KB,
// so two workgroups share a compute unit and one's start-up (sequence bounds, Q)
// overlaps the other's streaming.  (Four stages in 128 KB measured no faster.)
// fp32 tiles go through registers: one stage.
template <typename T>
constexpr int dec_stages() {
  return sizeof(T) == 2 ? 2 : 1;
}

// Key tiles [tb, te) that the rows of one sequence can see (their union is one interval).
struct TileRange {
  int tb, te;
};
__device__ inline TileRange visible_tiles(int nq, int nk, int causal, int window) {
  if (nq <= 0) return {0, 0};
  const int off = nk - nq;
  const Span first = keys_of_row(0, off, nk, causal, window);
  const Span last = keys_of_row(nq - 1, off, nk, causal, window);
  const int klo = first.lo, khi = last.lo + (int)last.len;
  if (khi <= klo) return {0, 0};
  return {klo / kDecBN, (khi + kDecBN - 1) / kDecBN};
}

// D: head dim (64 or 128).
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_partial_kernel(DecodeArgs a) {
  using M = Mfma<T>;
  using Frag = typename M::Frag;
  constexpr int E = M::E, KS = M::KS;
  constexpr int NQ = D / KS;       // operand steps over the head dim
  constexpr int NP = kDecBN / KS;  // operand steps over the keys of a tile
  constexpr int TILE = tile_elems_d<T, D>(kDecBN);
  constexpr int STAGES = dec_stages<T>();
  constexpr int MT = kDecBN / 32;  // 32-key blocks per tile
  __shared__ __attribute__((aligned(16))) T smem[kDecWaves * STAGES * 2 * TILE];

  const FwdArgs& f = a.f;
  // Workgroups are dealt to the 8 XCDs by linear index (x + X y) mod 8.  Rotating the
  // (sequence, kv-head block) column by the chunk row spreads each sequence's chunks
  // over consecutive XCDs; without it a column (and so a whole sequence) stays on one
  // XCD, and with ragged lengths the XCD holding the longest ones finishes last.
  const int col = (int)((blockIdx.x + blockIdx.y) % gridDim.x);
  const int gblocks = f.hkv / a.hw;
  const int b = col / gblocks;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = (col % gblocks) * a.hw + w;  // this wavefront's kv head
  const int h = lane >> 5, c = lane & 31;
  const int G = f.hq / f.hkv;

  const SeqBounds sq = seq_bounds(f.cu_q, b, f.total_q);
  const SeqBounds sk = seq_bounds(f.cu_k, b, f.total_k);
  const int nq = sq.len, nk = sk.len, off = nk - nq;
  const TileRange tr = visible_tiles(nq, nk, f.causal, f.window);
  // (clamped to the grid: a sequence longer than max_seqlen_k is only partly computed)
  const int nchunks = min(max((tr.te - tr.tb + a.chunk - 1) / a.chunk, 1), a.max_chunks);
  const int ci = blockIdx.y;
  if (nq == 0 || ci >= nchunks) return;  // uniform over the workgroup
  const int t0 = min(tr.tb + ci * a.chunk, tr.te), t1 = min(t0 + a.chunk, tr.te);

  // Column c: query head g*G + c % G, row c / G (valid while the row exists; the
  // workspace holds G * max_seqlen_q columns).
  const int col_row = c / G, col_head = g * G + c % G;
  const bool col_ok = c < G * (kDecCols / G) && col_row < nq && c < a.cols;
  Span keys = keys_of_row(col_row, off, nk, f.causal, f.window);
  if (!col_ok) keys.len = 0u;

  // Q fragments (B operand of S^T = K Q^T): lane owns column c, d = KS*s + E*h + e.
  // Loaded after the first tiles' loads are issued, so the two round trips overlap.
  Frag qf[NQ];
  auto load_q = [&]() __attribute__((always_inline)) {
    const T* src = static_cast<const T*>(f.q) + ((size_t)(sq.start + (col_ok ? col_row : 0)) * f.hq +
                                                 (col_ok ? col_head : 0)) * D;
#pragma unroll
    for (int s = 0; s < NQ; ++s) qf[s] = global_frag<T>(src + KS * s + E * h, col_ok);
    vmem_drain();  // the Q loads (and anything issued before them) are done
  };
  const float sl2 = f.scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[D / 32];  // O^T: [D x 32 columns]
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[t][r] = 0.f;

  const size_t kv_row = (size_t)f.hkv * D;
  T* const stage0 = smem + w * STAGES * 2 * TILE;  // [stage][K, V]
  FragAddr<T> fa;
  fa.init(lane);
  TileLoaderD<T, kDecBN, 64, D> kld, vld;  // each wavefront moves its own tiles
  kld.init(static_cast<const T*>(f.k) + (size_t)sk.start * kv_row + g * D, kv_row, nk, lane);
  vld.init(static_cast<const T*>(f.v) + (size_t)sk.start * kv_row + g * D, kv_row, nk, lane);

  // One key tile against the 32 columns: scores, mask, online softmax, P V.
  auto tile = [&](int t, const T* Ks, const T* Vs) __attribute__((always_inline)) {
    f32x16 st[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st[mt][r] = 0.f;
#pragma unroll
      for (int s = 0; s < NQ; ++s) st[mt] = M::mma(frag_row<T, kDecBN>(fa, Ks, mt, s), qf[s], st[mt]);
    }
    // Mask to the column's visible keys (key of register r: t*BN + 4h + 32mt + 8(r/4) + r%4).
    const int k0 = t * kDecBN + 4 * h;
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
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
    for (int t2 = 0; t2 < D / 32; ++t2)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[t2][r] *= alpha;
    m_run = m_new;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) st[mt][r] = fast_exp2(fmaf(st[mt][r], sl2, neg_m));
    // The normaliser sums the float32 P before it is rounded into operands, as the
    // training forward does, so the two paths differ only in summation order.
    float tsum = 0.f;
#pragma unroll
    for (int s = 0; s < NP; ++s) {
      if constexpr (sizeof(T) == 2) {
        const int r0 = 8 * (s % 2);
        const f32x16& x = st[s / 2];
        tsum += ((x[r0] + x[r0 + 1]) + (x[r0 + 2] + x[r0 + 3])) + ((x[r0 + 4] + x[r0 + 5]) + (x[r0 + 6] + x[r0 + 7]));
      }
      const Frag pf = pack_frag<T>(st, s);
      if constexpr (sizeof(T) != 2) tsum = frag_sum<T>(pf, tsum);
#pragma unroll
      for (int md = 0; md < D / 32; ++md) oacc[md] = M::mma(frag_col<T, kDecBN>(fa, Vs, md, s), pf, oacc[md]);
    }
    l_run += tsum;
  };

  // Each wavefront moves its own tiles and waits only for its own loads (no
  // workgroup barrier).  The waits are asm with a memory clobber, which also keeps
  // the compiler from moving a tile's LDS reads above them; a stage is refilled
  // only after the MFMAs that read it were issued (their operands had returned).
  if constexpr (STAGES > 1) {
    constexpr int PER_TILE = 2 * decltype(kld)::N;  // DMA instructions per tile (K and V)
    auto stage = [&](int i) __attribute__((always_inline)) { return stage0 + (i % STAGES) * 2 * TILE; };
    auto issue = [&](int t, T* dst) __attribute__((always_inline)) {
      kld.issue(t * kDecBN, dst);
      vld.issue(t * kDecBN, dst + TILE);
    };
#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p)
      if (t0 + p < t1) issue(t0 + p, stage(p));
    load_q();
    for (int t = t0; t < t1; ++t) {
      const int i = t - t0;
      // Refill the stage of tile t - 1, whose LDS reads have all returned.
      if (t + STAGES - 1 < t1) issue(t + STAGES - 1, stage(i + STAGES - 1));
      // Wait until tile t has landed: allow the DMAs of the tiles issued after it.
      const int ahead = min(STAGES - 1, t1 - 1 - t);
      static_assert(STAGES <= 4 && 3 * PER_TILE < 64, "wait counts below");
      if (ahead >= 3)
        wait_vmcnt<3 * PER_TILE>();
      else if (ahead == 2)
        wait_vmcnt<2 * PER_TILE>();
      else if (ahead == 1)
        wait_vmcnt<PER_TILE>();
      else
        wait_vmcnt<0>();
      const T* const cur = stage(i);
      tile(t, cur, cur + TILE);
    }
  } else {
    load_q();
    for (int t = t0; t < t1; ++t) {
      kld.issue(t * kDecBN, stage0);
      vld.issue(t * kDecBN, stage0 + TILE);
      kld.finish();
      vld.finish();
      wait_vmcnt<0>();
      tile(t, stage0, stage0 + TILE);
    }
  }
  const float l_col = halves_sum(l_run);
  if (!col_ok) return;

  // Lane (c, h) holds O^T rows d = 32 md + 8 r4 + 4 h + e (e = 0..3) of column c.
  if (nchunks == 1) {
    // The whole visible range was this chunk: add the sink's mass, normalise, write.
    const float sink2 = f.sinks[col_head] * kLog2e;
    const float mm = fmaxf(m_run, sink2);
    float o_sc = 0.f, l_tot = 0.f;
    if (mm > -INFINITY) {
      o_sc = m_run == -INFINITY ? 0.f : fast_exp2(m_run - mm);
      l_tot = l_col * o_sc + (sink2 > -INFINITY ? fast_exp2(sink2 - mm) : 0.f);
    }
    const float inv = l_tot > 0.f ? o_sc / l_tot : 0.f;
    T* dst = static_cast<T*>(f.o) + ((size_t)(sq.start + col_row) * f.hq + col_head) * D;
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
      f.lse[(size_t)col_head * f.total_q + sq.start + col_row] =
          l_tot > 0.f ? (mm + fast_log2(l_tot)) * kLn2 : -INFINITY;
    return;
  }
  // Partial of this chunk: column slot c of (sequence, kv head, chunk).
  const size_t slot = ((size_t)(b * f.hkv + g) * a.max_chunks + ci) * a.cols + c;
  float* po = a.part_o + slot * D;
#pragma unroll
  for (int md = 0; md < D / 32; ++md)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = 32 * md + crow(4 * r4, h);
      *reinterpret_cast<f32x4*>(po + d0) =
          f32x4{oacc[md][4 * r4], oacc[md][4 * r4 + 1], oacc[md][4 * r4 + 2], oacc[md][4 * r4 + 3]};
    }
  if (h == 0) *reinterpret_cast<float2*>(a.part_ml + 2 * slot) = float2{m_run, l_col};
}

// One workgroup per (sequence, kv head); a wavefront per column (query head, new
// row), lane = d (and d + 64 when D = 128).  The column's chunk statistics are
// wavefront-uniform.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  constexpr int DL = D / 64;  // values of d per lane
  const FwdArgs& f = a.f;
  const int b = blockIdx.x / f.hkv, g = blockIdx.x % f.hkv;
  const int G = f.hq / f.hkv;
  const SeqBounds sq = seq_bounds(f.cu_q, b, f.total_q);
  const SeqBounds sk = seq_bounds(f.cu_k, b, f.total_k);
  const TileRange tr = visible_tiles(sq.len, sk.len, f.causal, f.window);
  const int nchunks = min((tr.te - tr.tb + a.chunk - 1) / a.chunk, a.max_chunks);
  if (nchunks <= 1) return;  // finished by the partial kernel
  const int ncols = min(G * min(sq.len, kDecCols / G), a.cols);
  const int d = threadIdx.x & 63;
  const int nw = blockDim.x >> 6;
  const size_t base = (size_t)(b * f.hkv + g) * a.max_chunks * a.cols;  // slot of chunk 0, column 0
  for (int cc = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); cc < ncols; cc += nw) {
    const int row = cc / G, head = g * G + cc % G;
    const float* ml = a.part_ml + 2 * (base + cc);      // chunk ch at 2 * ch * cols
    const float* po = a.part_o + (base + cc) * D + d;  // chunk ch at ch * cols * D
    const size_t mstride = 2 * (size_t)a.cols, ostride = (size_t)a.cols * D;
    // Running (max M, sum l, output o), seeded with the sink's mass; chunks are
    // merged in order, U at a time: the U chunks' values are loaded together (one
    // round trip), then folded in.
    const float sink2 = f.sinks[head] * kLog2e;
    float mm = sink2, l = sink2 > -INFINITY ? 1.f : 0.f, o[DL];
#pragma unroll
    for (int j = 0; j < DL; ++j) o[j] = 0.f;
    constexpr int U = 16;
    for (int c0 = 0; c0 < nchunks; c0 += U) {
      float ms[U], ls[U], os[U][DL];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool ok = c0 + u < nchunks;
        ms[u] = ok ? ml[(c0 + u) * mstride] : -INFINITY;
        ls[u] = ok ? ml[(c0 + u) * mstride + 1] : 0.f;
#pragma unroll
        for (int j = 0; j < DL; ++j) os[u][j] = ok ? po[(c0 + u) * ostride + 64 * j] : 0.f;
      }
      float bm = mm;
#pragma unroll
      for (int u = 0; u < U; ++u) bm = fmaxf(bm, ms[u]);
      if (bm == -INFINITY) continue;  // nothing seen yet, no sink
      const float sc = mm == -INFINITY ? 0.f : fast_exp2(mm - bm);
      l *= sc;
#pragma unroll
      for (int j = 0; j < DL; ++j) o[j] *= sc;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // a chunk in which this row sees no key has ms = -inf, l = 0, O = 0
        const float e = ms[u] == -INFINITY ? 0.f : fast_exp2(ms[u] - bm);
        l += ls[u] * e;
#pragma unroll
        for (int j = 0; j < DL; ++j) o[j] += os[u][j] * e;
      }
      mm = bm;
    }
    const size_t orow = (size_t)(sq.start + row) * f.hq + head;
#pragma unroll
    for (int j = 0; j < DL; ++j)
      static_cast<T*>(f.o)[orow * D + d + 64 * j] = from_f32<T>(l > 0.f ? o[j] / l : 0.f);
    if (d == 0) f.lse[(size_t)head * f.total_q + sq.start + row] = l > 0.f ? (mm + fast_log2(l)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------- fixed scratch
// The workspace of the allocation-free decoding entry point: one copy of this array
// per GPU (each device that loads the library holds its own, until the process
// ends).  Host code never passes the array's name to a kernel (on the host it is a
// stand-in, not a device address): decode_scratch() looks the device address up
// once per device and keeps it.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // the current device's copy
    if (e != hipSuccess) return e;
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255) != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode_partial(const DecodeArgs& a, int fp32, hipStream_t stream) {
  dim3 grid(a.f.num_seqs * (a.f.hkv / a.hw), a.max_chunks);
  dim3 block(64 * a.hw);
  if (a.f.d == 128) {
    if (fp32)
      hipLaunchKernelGGL((decode_partial_kernel<float, 128>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((decode_partial_kernel<bf16, 128>), grid, block, 0, stream, a);
  } else {
    if (fp32)
      hipLaunchKernelGGL((decode_partial_kernel<float, 64>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((decode_partial_kernel<bf16, 64>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeArgs& a, int fp32, hipStream_t stream) {
  if (a.max_chunks <= 1) return hipSuccess;  // every sequence is finished by the partial kernel
  dim3 grid(a.f.num_seqs * a.f.hkv);
  if (a.f.d == 128) {
    if (fp32)
      hipLaunchKernelGGL((decode_merge_kernel<float, 128>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_merge_kernel<bf16, 128>), grid, dim3(256), 0, stream, a);
  } else {
    if (fp32)
      hipLaunchKernelGGL((decode_merge_kernel<float, 64>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_merge_kernel<bf16, 64>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace attn_sink
