// Device-side building blocks shared by the forward and backward kernels (gfx950 / CDNA4).
//
// Matrix-core convention used everywhere: one wavefront (64 lanes) runs
// v_mfma_f32_32x32x16_bf16 (bf16) or v_mfma_f32_32x32x2_f32 (fp32) on 32x32 tiles.
// With l = lane, h = l / 32 (lane half) and c = l % 32:
//   A operand (M x K): lane holds row c,    k-slots [E*h, E*h + E) of the step
//   B operand (K x N): lane holds column c, k-slots [E*h, E*h + E) of the step
//   C/D (32 x 32 fp32, 16 registers): register r of lane l holds
//       row 8*(r/4) + 4*h + (r%4), column c
// E = 8 elements per lane for bf16 (K = 16 per instruction), E = 1 for fp32 (K = 2).
// A contraction only needs A and B to agree on which logical k each (h, slot)
// carries, so when a C tile is fed back as an operand, its row index becomes the
// k index through the permutation kc(f, h) below.
//
// LDS tiles are row-major with 64 columns.  bf16 tiles swizzle their 16-byte
// chunks (chunk c of row r is stored at c ^ swz(r)).  The LDS has 64 four-byte
// banks and serves a ds_read_b128 sixteen lanes per clock, so the sixteen rows a
// 16-lane group reads at one logical chunk must land on sixteen distinct 16-byte
// bank groups: a row pair (2j, 2j+1) spans all 64 banks, and swz must take eight
// distinct values over the even (and over the odd) rows of any aligned 16 rows.
// The transposing reads (ds_read_b64_tr_b16, four rows x 32 bytes per 16 lanes)
// additionally want rows r and r+2 of an aligned quad in different halves of the
// row: swz(r) = 4 * bit1(r) + bits2..3(r) satisfies both.  fp32 tiles use a padded
// stride of 65 words.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn_sink {

constexpr int kD = 64;  // columns of one LDS tile block; head dims are multiples of it (64, 128)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Mfma;

template <>
struct Mfma<bf16> {
  static constexpr int E = 8;    // elements per lane per operand
  static constexpr int KS = 16;  // contraction length of one instruction
  using Frag = bf16x8;
  __device__ static inline f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mfma<float> {
  static constexpr int E = 1;
  static constexpr int KS = 2;
  using Frag = float;
  __device__ static inline f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Row of C register r in lane half h (0..31).
__device__ __host__ constexpr int crow(int r, int h) { return 8 * (r / 4) + 4 * h + (r % 4); }

// When the 32 registers of two stacked C tiles (tile = f / 16, register = f % 16)
// feed a contraction over their row index, slot e of step s takes flat register
// f = E*s + e; this is the logical k (0..63) it stands for, in lane half h.
__device__ __host__ constexpr int kc(int f, int h) { return 32 * (f / 16) + crow(f % 16, h); }

__device__ inline float to_f32(bf16 x) { return (float)x; }
__device__ inline float to_f32(float x) { return x; }
template <typename T>
__device__ inline T from_f32(float x) { return (T)x; }  // bf16: round to nearest even

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------- LDS tile layout
template <typename T>
struct Tile;

template <>
struct Tile<bf16> {
  static constexpr int ELEMS_PER_ROW = 64;
  __device__ static inline int swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
  // element offset of (row, col); col % 4 == 0 keeps a 4-element run inside one chunk
  __device__ static inline int off(int r, int c) { return r * 64 + ((((c >> 3) ^ swz(r)) << 3) | (c & 7)); }
};

template <>
struct Tile<float> {
  static constexpr int ELEMS_PER_ROW = 65;
  __device__ static inline int off(int r, int c) { return r * 65 + c; }
};

template <typename T>
constexpr int tile_elems(int rows) {
  return rows * Tile<T>::ELEMS_PER_ROW;
}

// A tile of D columns (D = 64 or 128) is stored as D / 64 consecutive 64-column
// blocks, each a `rows` x 64 tile in the layout above, so every operand read and
// DMA pattern stays that of the 64-column tile.
template <typename T, int D>
constexpr int tile_elems_d(int rows) {
  return (D / kD) * tile_elems<T>(rows);
}

// Operand whose lane holds row `row` and k-slots [col, col + E) of a tile
// (the k index runs along the row: contiguous).
template <typename T>
__device__ inline typename Mfma<T>::Frag lds_row_frag(const T* tile, int row, int col) {
  return *reinterpret_cast<const typename Mfma<T>::Frag*>(tile + Tile<T>::off(row, col));
}

// Operand whose lane holds COLUMN m0 + lane%32 of a tile and, in its k-slots, rows
// of the tile: rows kc(E*s + e, h) when `perm` (a C tile fed back as operand),
// else KS*s + E*h + e.  bf16 uses two transposing reads (ds_read_b64_tr_b16): in
// each 16-lane group, source lane u reads row r0 + u/4 at columns c0 + 4*(u%4) ..+3,
// and output lane t receives rows r0 .. r0+3 at column c0 + t.
template <typename T>
__device__ inline typename Mfma<T>::Frag lds_col_frag(const T* tile, int m0, int s, int lane, bool perm) {
  const int h = lane >> 5;
  if constexpr (Mfma<T>::E == 8) {
    const int g = lane >> 4, t = lane & 15;
    const int r0 = perm ? kc(8 * s, h) : 16 * s + 8 * h;
    const int r1 = perm ? kc(8 * s + 4, h) : 16 * s + 8 * h + 4;
    const int c = m0 + 16 * (g & 1) + 4 * (t & 3);
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + Tile<bf16>::off(r0 + (t >> 2), c)));
    i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + Tile<bf16>::off(r1 + (t >> 2), c)));
    bf16x4 ab = __builtin_bit_cast(bf16x4, a), bb = __builtin_bit_cast(bf16x4, b);
    return bf16x8{ab[0], ab[1], ab[2], ab[3], bb[0], bb[1], bb[2], bb[3]};
  } else {
    const int row = perm ? kc(s, h) : 2 * s + h;
    return tile[Tile<float>::off(row, m0 + (lane & 31))];
  }
}

// The same two fragment kinds through per-lane byte offsets computed once per
// kernel.  Every fragment a kernel reads from a 64-column tile is one of eight
// per-lane offsets plus a compile-time constant (the swizzle depends on row bits
// 1..3 only, so moving by 16 or 32 rows keeps it), which lets a read of a tile at a
// compile-time LDS address use the instruction's immediate offset and no address
// arithmetic at all.  The offsets are pinned (opaque to the optimiser) so they are
// kept in eight VGPRs rather than recomputed inside the loops.
//   row(tile, mt, s): lds_row_frag(tile, 32*mt + c, KS*s + E*h)
//   col(tile, md, s): lds_col_frag(tile, 32*md, s, lane, perm = true)
template <typename T>
struct FragAddr;

template <>
struct FragAddr<bf16> {
  uint32_t row_[4];     // bytes of (row c, logical column 16 s + 8 h), s = 0..3
  uint32_t col_[2][2];  // [j][md]: bytes of (row 8 j + 4 h + t/4, column 32 md + 16 (g&1) + 4 (t&3))
  // pin = false leaves the offsets to the optimiser, which may then recompute them
  // rather than hold eight registers (a kernel at a tight register budget).
  __device__ inline void init(int lane, bool pin = true) {
    const int h = lane >> 5, c = lane & 31, g = lane >> 4, t = lane & 15;
#pragma unroll
    for (int s = 0; s < 4; ++s) row_[s] = 2u * (uint32_t)Tile<bf16>::off(c, 16 * s + 8 * h);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int md = 0; md < 2; ++md)
        col_[j][md] = 2u * (uint32_t)Tile<bf16>::off(8 * j + 4 * h + (t >> 2), 32 * md + 16 * (g & 1) + 4 * (t & 3));
    if (!pin) return;
#pragma unroll
    for (int s = 0; s < 4; ++s) asm volatile("" : "+v"(row_[s]));
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int md = 0; md < 2; ++md) asm volatile("" : "+v"(col_[j][md]));
  }
  __device__ inline bf16x8 row(const bf16* tile, int mt, int s) const {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(tile) + row_[s] + mt * (32 * 64 * 2));
  }
  // rows kc(8 s, h) + t/4 = 16 s + 4 h + t/4 and kc(8 s + 4, h) + t/4 = that + 8
  __device__ inline bf16x8 col(const bf16* tile, int md, int s) const {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const char* base = reinterpret_cast<const char*>(tile) + s * (16 * 64 * 2);
    i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + col_[0][md]));
    i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + col_[1][md]));
    bf16x4 ab = __builtin_bit_cast(bf16x4, a), bb = __builtin_bit_cast(bf16x4, b);
    return bf16x8{ab[0], ab[1], ab[2], ab[3], bb[0], bb[1], bb[2], bb[3]};
  }
};

template <>
struct FragAddr<float> {
  int lane_;
  __device__ inline void init(int lane, bool = true) { lane_ = lane; }
  __device__ inline float row(const float* tile, int mt, int s) const {
    return lds_row_frag<float>(tile, 32 * mt + (lane_ & 31), 2 * s + (lane_ >> 5));
  }
  __device__ inline float col(const float* tile, int md, int s) const {
    return lds_col_frag<float>(tile, 32 * md, s, lane_, true);
  }
};

// The two fragment kinds on a tile of ROWS rows and D columns (tile_elems_d): step s
// of the contraction over the columns (row fragments) or column block md of 32
// (transposed fragments) picks its 64-column block at a compile-time offset.
template <typename T, int ROWS>
__device__ inline typename Mfma<T>::Frag frag_row(const FragAddr<T>& fa, const T* tile, int mt, int s) {
  constexpr int PER = kD / Mfma<T>::KS;  // steps per 64-column block
  return fa.row(tile + (s / PER) * tile_elems<T>(ROWS), mt, s % PER);
}
template <typename T, int ROWS>
__device__ inline typename Mfma<T>::Frag frag_col(const FragAddr<T>& fa, const T* tile, int md, int s) {
  return fa.col(tile + (md / 2) * tile_elems<T>(ROWS), md % 2, s);
}

// d = A B + c (bf16, 32x32x16) with c in registers distinct from d: the first
// step of an accumulation that starts from a non-zero seed kept elsewhere (the
// compiler would first copy the seed into d).  The leading s_nop covers a VALU
// write of A, B or c just before.  MFMAs that go on accumulating into d need no
// wait states; a VALU read of d must come after a later compiler-emitted MFMA
// on d (the compiler does not see this one's latency).  Not volatile: a volatile asm would be a
// scheduling boundary and pin the LDS operand reads around it.
__device__ inline f32x16 mma_seeded(bf16x8 a, bf16x8 b, const f32x16& c) {
  f32x16 d;
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// d = A B + c with the seed c kept in its own registers (first step of a seeded
// accumulation): bf16 through mma_seeded, fp32 through the builtin.
template <typename T>
__device__ inline f32x16 mma_first(typename Mfma<T>::Frag a, typename Mfma<T>::Frag b, const f32x16& c) {
  if constexpr (Mfma<T>::E == 8) {
    return mma_seeded(a, b, c);
  } else {
    return Mfma<T>::mma(a, b, c);
  }
}

// Pack flat registers [E*s, E*s + E) of two stacked C tiles into an operand.
template <typename T>
__device__ inline typename Mfma<T>::Frag pack_frag(const f32x16* c, int s) {
  if constexpr (Mfma<T>::E == 8) {
    const f32x16& t = c[s / 2];
    const int r0 = 8 * (s % 2);
    bf16x8 f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (bf16)t[r0 + e];
    return f;
  } else {
    return c[s / 16][s % 16];
  }
}

// max / sum of x over the two lane halves (lanes l and l ^ 32), via v_permlane32_swap.
__device__ inline float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// acc + sum of the E elements of an operand fragment (bf16: four v_dot2 with (1, 1)).
template <typename T>
__device__ inline float frag_sum(typename Mfma<T>::Frag f, float acc) {
  if constexpr (Mfma<T>::E == 8) {
    const bf16x2 ones = {(bf16)1.f, (bf16)1.f};
#pragma unroll
    for (int e = 0; e < 8; e += 2) acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{f[e], f[e + 1]}, ones, acc, false);
    return acc;
  } else {
    return acc + f;
  }
}

// acc + the dot product of two operand fragments (bf16: four v_dot2).
template <typename T>
__device__ inline float frag_dot(typename Mfma<T>::Frag a, typename Mfma<T>::Frag b, float acc) {
  if constexpr (Mfma<T>::E == 8) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{a[e], a[e + 1]}, bf16x2{b[e], b[e + 1]}, acc, false);
    return acc;
  } else {
    return fmaf(a, b, acc);
  }
}

// ---------------------------------------------------------------- global <-> LDS staging
// A tile of `ROWS` rows x 64 columns of one head, moved as 16-byte chunks (CPR per
// row) with raw buffer loads through one descriptor that covers exactly the
// sequence's rows of this head.  The whole byte offset of a chunk (the tile's first
// row plus the lane's row and column) goes in the VGPR offset: the raw-buffer range
// check compares that offset (not the scalar one) with the descriptor's size, so
// chunks past the last row read as zero and nothing beyond the sequence is touched.
// Offsets are 32-bit: the caller guarantees (nrows + 128) * row_bytes < 2^32, and
// tiles start at a row below nrows.  Where registers are tight, issue_rebased()
// moves the tile's first row into the descriptor instead (base + row0 rows, sized
// to the rows left), which costs scalar instructions and no vector register.
constexpr int kBufferWord3 = 0x00020000;  // gfx9-family raw buffer descriptor, dword 3

__device__ inline __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}

template <typename T, int ROWS, int THREADS>
struct Stager {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int CPR = kD / VEC;
  static constexpr int N = ROWS * CPR / THREADS;  // chunks per thread
  static_assert(ROWS * CPR % THREADS == 0, "tile must split evenly over the threads");
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t row_bytes;
  uint32_t voff[N];
  uint4 reg[N];
  // base: element (row 0, column 0) of the head; rows are row_stride elements apart;
  // nrows rows are readable.
  __device__ inline void init(const T* base, size_t row_stride, int nrows, int tid) {
    row_bytes = (uint32_t)(row_stride * sizeof(T));
    rsrc = rows_rsrc(base, (uint32_t)nrows * row_bytes);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int ch = tid + THREADS * i;
      voff[i] = (uint32_t)(ch / CPR) * row_bytes + (uint32_t)(ch % CPR) * 16u;
    }
  }
  // Load the tile whose first row is row0 (rows >= nrows read as zero).
  __device__ inline void load(int row0) {
    const uint32_t toff = (uint32_t)row0 * row_bytes;
#pragma unroll
    for (int i = 0; i < N; ++i)
      reg[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff[i] + toff, 0, 0));
  }
  __device__ inline void store(T* tile, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int ch = tid + THREADS * i;
      const int r = ch / CPR, col = ch % CPR;
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<uint4*>(tile + Tile<T>::off(r, col * VEC)) = reg[i];
      } else {
        const float* f = reinterpret_cast<const float*>(&reg[i]);
#pragma unroll
        for (int e = 0; e < 4; ++e) tile[Tile<T>::off(r, col * VEC + e)] = f[e];
      }
    }
  }
};

// Buffer load whose data goes straight to LDS: lane i's bytes land at LDS byte
// address lds + size * i.  Issued through inline asm on purpose: the compiler
// tracks its own LDS DMA builtin as an LDS write it cannot disambiguate from the
// transposing LDS reads, and then waits for every outstanding DMA (the prefetch
// of the next tile) before the first such read of the current tile.  The caller
// orders the DMA explicitly (s_waitcnt vmcnt(0) + barrier before the data is
// read), and the compiler's own vmcnt waits stay correct (only more conservative)
// because vector-memory loads retire in order.
__device__ inline uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// The scalar offset is 0: the whole offset is in voff, where the range check sees it.
__device__ inline void lds_dma_b128(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}
__device__ inline void lds_dma_b32(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}

// Wait for every outstanding vector-memory load.  Called once after a kernel's
// prologue (whose waits are conditional): it tells the compiler that the register
// loads issued so far (fragments kept in registers for the whole loop) are done,
// so it places no vmcnt wait for them inside the loop, where it would also wait
// for the asm tile DMAs in flight.
__device__ inline void vmem_drain() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Wait until at most N of this wavefront's vector-memory instructions are in flight
// (N < 64), as asm with a memory clobber: the compiler neither moves memory accesses
// across it nor knows of the asm DMAs it waits for.
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Tile loader with one interface for both element types: issue(row0, tile) starts
// moving rows [row0, row0 + ROWS) of the head into LDS tile `tile`, finish() makes
// sure they have arrived (the caller then synchronises the workgroup).
//  * bf16: direct global -> LDS buffer loads (no registers, no LDS write
//    instructions).  One wavefront instruction fills 64 consecutive 16-byte LDS
//    slots; each lane fetches the global chunk that the swizzled layout stores in
//    its slot.
//  * fp32: through registers (the padded fp32 layout is not 16-byte aligned).
template <typename T, int ROWS, int THREADS>
struct TileLoader;

template <int ROWS, int THREADS>
struct TileLoader<bf16, ROWS, THREADS> {
  static constexpr int N = ROWS * 8 / THREADS;  // 16-byte slots per thread
  static_assert(ROWS * 8 % THREADS == 0, "tile must split evenly over the threads");
  __amdgpu_buffer_rsrc_t rsrc;
  const bf16* base_;
  int nrows_;
  uint32_t row_bytes;
  uint32_t voff[N];
  int first_slot;  // first LDS slot (of 64) written by this wavefront's instructions
  // Tile row r is array row row0 + r.
  __device__ inline void init(const bf16* base, size_t row_stride, int nrows, int tid) {
    init_rows(base, row_stride, nrows, tid, 0, 0u);
  }
  // Packed rows: tile row r is array row row0 + (r >> lg), plus (r & (2^lg - 1)) *
  // sub_bytes within it (the heads of one position); rows >= nrows read as zero.
  __device__ inline void init_rows(const bf16* base, size_t row_stride, int nrows, int tid, int lg,
                                   uint32_t sub_bytes) {
    base_ = base;
    nrows_ = nrows;
    row_bytes = (uint32_t)(row_stride * sizeof(bf16));
    rsrc = rows_rsrc(base, (uint32_t)nrows * row_bytes);
    const int lane = tid & 63;
    first_slot = __builtin_amdgcn_readfirstlane(tid >> 6) * N * 64;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int slot = first_slot + n * 64 + lane;  // LDS byte offset 16 * slot in the tile
      const int r = slot >> 3, pc = slot & 7;
      const int col_chunk = pc ^ Tile<bf16>::swz(r);  // slot (r, pc) holds logical chunk pc ^ swz(r)
      voff[n] = (uint32_t)(r >> lg) * row_bytes + (uint32_t)(r & ((1 << lg) - 1)) * sub_bytes +
                (uint32_t)col_chunk * 16u;
    }
  }
  __device__ inline void issue(int row0, bf16* tile) {
#if defined(__HIP_DEVICE_COMPILE__)  // device-only asm
    const uint32_t toff = (uint32_t)row0 * row_bytes;
#pragma unroll
    for (int n = 0; n < N; ++n) lds_dma_b128(rsrc, voff[n] + toff, lds_address(tile + (first_slot + n * 64) * 8));
#endif
  }
  __device__ inline void issue_rebased(int row0, bf16* tile) {
#if defined(__HIP_DEVICE_COMPILE__)
    const char* p = reinterpret_cast<const char*>(base_) + (size_t)row0 * row_bytes;
    const __amdgpu_buffer_rsrc_t r = rows_rsrc(p, (uint32_t)max(nrows_ - row0, 0) * row_bytes);
#pragma unroll
    for (int n = 0; n < N; ++n) lds_dma_b128(r, voff[n], lds_address(tile + (first_slot + n * 64) * 8));
#endif
  }
  __device__ inline void finish() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)
};

template <int ROWS, int THREADS>
struct TileLoader<float, ROWS, THREADS> {
  static constexpr int N = Stager<float, ROWS, THREADS>::N;  // register loads per thread
  Stager<float, ROWS, THREADS> st;
  float* dst;
  int tid_;
  __device__ inline void init(const float* base, size_t row_stride, int nrows, int tid) {
    st.init(base, row_stride, nrows, tid);
    tid_ = tid;
  }
  __device__ inline void issue(int row0, float* tile) {
    st.load(row0);
    dst = tile;
  }
  __device__ inline void issue_rebased(int row0, float* tile) { issue(row0, tile); }
  __device__ inline void finish() { st.store(dst, tid_); }
};

// A tile of ROWS rows and D columns of one head (tile_elems_d layout): one 64-column
// loader per column block.  N: vector-memory instructions per thread and tile.
template <typename T, int ROWS, int THREADS, int D>
struct TileLoaderD {
  using Sub = TileLoader<T, ROWS, THREADS>;
  static constexpr int BLOCKS = D / kD;
  static constexpr int N = BLOCKS * Sub::N;
  Sub sub[BLOCKS];
  __device__ inline void init(const T* base, size_t row_stride, int nrows, int tid) {
#pragma unroll
    for (int i = 0; i < BLOCKS; ++i) sub[i].init(base + kD * i, row_stride, nrows, tid);
  }
  // Packed rows (bf16 only): see TileLoader<bf16>::init_rows.
  __device__ inline void init_rows(const T* base, size_t row_stride, int nrows, int tid, int lg, uint32_t sub_bytes) {
#pragma unroll
    for (int i = 0; i < BLOCKS; ++i) sub[i].init_rows(base + kD * i, row_stride, nrows, tid, lg, sub_bytes);
  }
  __device__ inline void issue(int row0, T* tile) {
#pragma unroll
    for (int i = 0; i < BLOCKS; ++i) sub[i].issue(row0, tile + i * tile_elems<T>(ROWS));
  }
  __device__ inline void issue_rebased(int row0, T* tile) {
#pragma unroll
    for (int i = 0; i < BLOCKS; ++i) sub[i].issue_rebased(row0, tile + i * tile_elems<T>(ROWS));
  }
  __device__ inline void finish() {
#pragma unroll
    for (int i = 0; i < BLOCKS; ++i) sub[i].finish();
  }
};

// 64 consecutive floats of one row-statistics array moved straight into LDS by one
// wavefront instruction (lane i -> float i); rows past `nrows` read as zero.
struct RowLoader {
  __amdgpu_buffer_rsrc_t rsrc;
  __device__ inline void init(const float* base, int nrows) { rsrc = rows_rsrc(base, (uint32_t)nrows * 4u); }
  // Call from one whole wavefront; finish with the tile loads' wait (vmcnt(0)).
  __device__ inline void issue(int row0, float* lds, int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
    lds_dma_b32(rsrc, (uint32_t)(row0 + lane) * 4u, lds_address(lds));
#endif
  }
  // Packed rows: lane i takes element row0 + (i >> lg) of sub-array i & (2^lg - 1),
  // the sub-arrays `sub_stride` floats apart (readable range: `nvals` floats).
  __device__ inline void init_packed(const float* base, int nvals) { rsrc = rows_rsrc(base, (uint32_t)nvals * 4u); }
  __device__ inline void issue_packed(int row0, float* lds, int lane, int lg, int sub_stride) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t i = (uint32_t)(lane & ((1 << lg) - 1)) * (uint32_t)sub_stride + (uint32_t)(row0 + (lane >> lg));
    lds_dma_b32(rsrc, i * 4u, lds_address(lds));
#endif
  }
};

// ---------------------------------------------------------------- misc
__device__ inline int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Sequence bounds with cu_seqlens clamped into [0, total].
struct SeqBounds {
  int start, len;
};
__device__ inline SeqBounds seq_bounds(const int* cu, int b, int total) {
  int a = clampi(cu[b], 0, total);
  int e = clampi(cu[b + 1], a, total);
  return {a, e - a};
}

// Key j visible to query i (local indices; off = n_k - n_q aligns the ends).
__device__ inline bool visible(int i, int j, int off, int nk, int causal, int window) {
  return (j < nk) & ((causal == 0) | (j <= i + off)) & ((window <= 0) | (j > i + off - window));
}

// The keys query row i sees form one interval, and so do the query rows that see
// key j (causal limit, window limit and sequence ends folded together).  A masked
// tile then costs one unsigned range check per element: (x - lo) < len.
struct Span {
  int lo;
  unsigned len;
};
__device__ inline Span keys_of_row(int i, int off, int nk, int causal, int window) {
  const int hi = causal ? min(i + off + 1, nk) : nk;      // key <= i + off, key < nk
  const int lo = window > 0 ? max(i + off - window + 1, 0) : 0;  // key > i + off - window
  return {lo, (unsigned)max(hi - lo, 0)};
}
__device__ inline Span rows_of_key(int j, int off, int nq, int nk, int causal, int window) {
  if (j >= nk) return {0, 0u};
  const int lo = causal ? max(j - off, 0) : 0;                   // i >= j - off
  const int hi = window > 0 ? min(j - off + window, nq) : nq;    // i < j - off + window, i < nq
  return {lo, (unsigned)max(hi - lo, 0)};
}
__device__ inline bool in_span(int x, Span s) { return (unsigned)(x - s.lo) < s.len; }

// Workgroups are dealt to the 8 XCDs round-robin (XCD = linear index % 8).  These
// maps turn the linear index of the workgroup's first grid dimension into
// (sequence, kv head, item within that kv head) such that every workgroup of kv
// head g runs on XCD g % 8: the query heads (or head splits) that read one kv
// head's K/V share an L2, and every XCD gets the same share of each sequence.
// `per_kv` items belong to each (sequence, kv head).  Falls back to plain order
// when the kv heads do not divide evenly over the XCDs.
struct XcdSlot {
  int seq, kv, item;
};
__device__ inline XcdSlot xcd_slot(int x, int num_kv, int per_kv) {
  XcdSlot r;
  if (num_kv % 8 == 0) {
    const int xcd = x % 8, j = x / 8;
    const int per_xcd = (num_kv / 8) * per_kv;  // items per sequence on one XCD
    r.seq = j / per_xcd;
    const int rem = j % per_xcd;
    r.kv = (rem / per_kv) * 8 + xcd;
    r.item = rem % per_kv;
  } else {
    r.item = x % per_kv;
    r.kv = (x / per_kv) % num_kv;
    r.seq = x / (per_kv * num_kv);
  }
  return r;
}

// Load E consecutive elements of a global row as an MFMA operand (zeros when !ok).
template <typename T>
__device__ inline typename Mfma<T>::Frag global_frag(const T* p, bool ok) {
  if constexpr (Mfma<T>::E == 8) {
    uint4 v = ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
    return __builtin_bit_cast(bf16x8, v);
  } else {
    return ok ? *p : 0.f;
  }
}

}  // namespace attn_sink
