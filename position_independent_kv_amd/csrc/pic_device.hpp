// Device-side building blocks for gfx950 (CDNA4): vector types, the MFMA
// instructions the attention kernels use, and their lane layouts.
//
// MFMA lane layout used throughout (wave64, 16x16 output tiles), with
// lane = 16 * grp + row16:
//   A operand (16 rows x K): lane holds A[row16][grp*KPL .. grp*KPL+KPL-1]
//   B operand (K x 16 cols): lane holds B[grp*KPL .. grp*KPL+KPL-1][row16]
//   C/D       (16 x 16)    : lane holds C[grp*4 + i][row16], i = 0..3
// KPL = 8 for v_mfma_f32_16x16x32_bf16 (K = 32), 1 for
// v_mfma_f32_16x16x4_f32 (K = 4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pic_common.hpp"

namespace pic {

template <typename T, int N>
using vec = T __attribute__((ext_vector_type(N)));

typedef __bf16 bf16;
typedef vec<float, 4> f32x4;

template <typename T>
struct Mma;

template <>
struct Mma<bf16> {
  static constexpr int KPL = 8;
  typedef vec<bf16, 8> Op;
  static __device__ __forceinline__ f32x4 run(Op a, Op b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ Op load(const bf16* p) {
    return *reinterpret_cast<const Op*>(p);
  }
  static __device__ __forceinline__ void store(bf16* p, const Op& v) {
    *reinterpret_cast<Op*>(p) = v;
  }
  static __device__ __forceinline__ float get(const Op& v, int e) { return (float)v[e]; }
  static __device__ __forceinline__ void set(Op& v, int e, float x) { v[e] = (bf16)x; }
  static __device__ __forceinline__ Op zero() {
    Op z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (bf16)0.0f;
    return z;
  }
  // 8 floats -> 8 bf16 (round to nearest even), converted two at a time
  static __device__ __forceinline__ Op pack(const float* f) {
    const vec<float, 8> v = {f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]};
    return __builtin_convertvector(v, Op);
  }
};

template <>
struct Mma<float> {
  static constexpr int KPL = 1;
  typedef float Op;
  static __device__ __forceinline__ f32x4 run(Op a, Op b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ Op load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, const Op& v) { *p = v; }
  static __device__ __forceinline__ float get(const Op& v, int) { return v; }
  static __device__ __forceinline__ void set(Op& v, int, float x) { v = x; }
  static __device__ __forceinline__ Op zero() { return 0.0f; }
  static __device__ __forceinline__ Op pack(const float* f) { return f[0]; }
};

template <typename T>
using OpT = typename Mma<T>::Op;

// v_mfma_f32_32x32x16_bf16.  Lane layout (lane = 32 * h + c, h in {0, 1}):
//   A (32 rows x 16): lane holds A[c][8h .. 8h+7]
//   B (16 x 32 cols): lane holds B[8h .. 8h+7][c]
//   C (32 x 32)     : lane holds C[8*(v/4) + 4h + v%4][c], v = 0..15
struct Mma32 {
  typedef vec<bf16, 8> Op;
  typedef vec<float, 16> Acc;
  static __device__ __forceinline__ Acc run(Op a, Op b, Acc c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

// Key (within a 32-key block) held in C row rho, chosen so that PV MFMA m's
// B operand -- K elements 8h..8h+7 -- is the lane's C values v = 8m..8m+7 and
// covers the 8 consecutive keys 16m + 8h .. 16m + 8h + 7.
__device__ __forceinline__ int key32(int rho) {
  const int j = rho >> 3, h = (rho >> 2) & 1, i = rho & 3;
  return 16 * (j >> 1) + 8 * h + 4 * (j & 1) + i;
}

// N contiguous elements, loaded / stored as one vector access when N > 1.
template <typename T, int N>
struct Run {
  typedef vec<T, N> V;
  static __device__ __forceinline__ V load(const T* p) { return *reinterpret_cast<const V*>(p); }
  static __device__ __forceinline__ void store(T* p, const V& v) { *reinterpret_cast<V*>(p) = v; }
};
template <typename T>
struct Run<T, 1> {
  typedef T V;
  static __device__ __forceinline__ V load(const T* p) { return *p; }
  static __device__ __forceinline__ void store(T* p, const V& v) { *p = v; }
};

template <typename T, int N>
__device__ __forceinline__ float elem(const typename Run<T, N>::V& v, int e) {
  if constexpr (N == 1) {
    return (float)v;
  } else {
    return (float)v[e];
  }
}
template <typename T, int N>
__device__ __forceinline__ void set_elem(typename Run<T, N>::V& v, int e, float x) {
  if constexpr (N == 1) {
    v = (T)x;
  } else {
    v[e] = (T)x;
  }
}

// Compile-time shape of the attention kernels for element type T and head size D.
template <typename T, int D>
struct Cfg {
  static constexpr int KPL = Mma<T>::KPL;
  static constexpr int KCH = 4 * KPL;          // d values per MFMA K-chunk
  static constexpr int NC = D / KCH;           // K-chunks over d
  static constexpr int NH = NC / 2;            // chunks holding the first half of d
  static constexpr int NT = (KPL == 8) ? 2 : 1;  // 16-key score tiles per step
  static constexpr int KSTEP = 16 * NT;        // keys per step
  static constexpr int NPV = 4 * NT / KPL;     // PV MFMAs per 16-row d tile per step
  static constexpr int ND = D / 16;            // 16-row d tiles of the output
  static constexpr int PAD = 16 / (int)sizeof(T);  // LDS row padding (16 bytes)
  static_assert(NC % 2 == 0, "rotate-half pairs chunk c with chunk c + NC/2");
};

// Key index (within a step) of score-tile t, tile row `row`.  Chosen so that
// the four C rows a lane holds in each tile, concatenated over the tiles, are
// the KPL consecutive keys its PV B operand needs (see the layout above).
template <int NT>
__device__ __forceinline__ int key_of(int t, int row) {
  return (row >> 2) * (4 * NT) + t * 4 + (row & 3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

}  // namespace pic
