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
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn_sink {

constexpr int kD = 64;  // head dim (the only one built)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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

// Fragment of E consecutive elements from LDS (16 B for bf16, 4 B for fp32).
template <typename T>
__device__ inline typename Mfma<T>::Frag lds_frag(const T* p) {
  return *reinterpret_cast<const typename Mfma<T>::Frag*>(p);
}

// Fragment whose slots e < 4 and e >= 4 come from two runs of 4 elements
// (bf16 only: two 8-byte reads).  For fp32 (E = 1) only p0 is used.
template <typename T>
__device__ inline typename Mfma<T>::Frag lds_frag_split(const T* p0, const T* p1) {
  if constexpr (Mfma<T>::E == 8) {
    bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
    bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  } else {
    return *p0;
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

// 16-byte global load / store helpers.
__device__ inline uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ inline void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

}  // namespace attn_sink
