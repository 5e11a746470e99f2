// Device-side helpers shared by the bf16 and fp8 attention kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace mi355attn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kBM = 128;      // query rows per workgroup, 32 per wave
constexpr int kBN = 64;       // keys per K/V tile
constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994530942f;

// Bijective remap of the hardware workgroup id so that ids dispatched to the
// same XCD (w % 8, round-robin dispatch) get consecutive logical ids, i.e. the
// query tiles of one head share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int w, int G) {
  const int q = G / kXcds, r = G % kXcds;
  const int x = w % kXcds, slot = w / kXcds;
  return x * q + min(x, r) + slot;
}

// v_permlane32_swap of a value with itself leaves, in every lane l, the pair
// {x[l % 32], x[l % 32 + 32]} (in some order): the two halves of one query row
// in the S^T accumulator layout.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Work item of one workgroup: (batch*head, query tile) and its key-tile range.
struct TileRange {
  int bh, q0, q_last, kt0, kt1;
};

// Masked problems (causal or windowed) visit their heaviest query tiles first.
__device__ __forceinline__ TileRange tile_range(int N, int nqt, int causal, int window) {
  TileRange t;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  t.bh = logical / nqt;
  const int qt = (causal || window >= 0) ? nqt - 1 - logical % nqt : logical % nqt;
  t.q0 = qt * kBM;
  t.q_last = min(N, t.q0 + kBM) - 1;
  // allowed keys of the whole query tile: [k_lo, k_hi)
  const int k_lo = window >= 0 ? max(0, t.q0 - window) : 0;
  const int k_hi = causal ? t.q_last + 1 : (window >= 0 ? min(N, t.q_last + window + 1) : N);
  t.kt0 = k_lo / kBN;
  t.kt1 = (k_hi + kBN - 1) / kBN;
  return t;
}

// Key tiles [ia, ib) inside [kt0, kt1) are "interior": every key of the tile is
// allowed for every query of the query tile, so they need no element mask.
// Tiles before ia and from ib on are "edge" tiles.
struct InteriorSpan {
  int ia, ib;
};
__device__ __forceinline__ InteriorSpan interior_span(const TileRange& t, int N, int causal,
                                                      int window) {
  const int lo_need = window >= 0 ? max(0, t.q_last - window) : 0;   // smallest key all rows allow
  int hi_need = N;                                                     // one past the largest
  if (causal) hi_need = min(hi_need, t.q0 + 1);
  else if (window >= 0) hi_need = min(hi_need, t.q0 + window + 1);
  InteriorSpan s;
  s.ia = min(max((lo_need + kBN - 1) / kBN, t.kt0), t.kt1);
  s.ib = min(max(hi_need / kBN, s.ia), t.kt1);
  return s;
}

// True if some (query, key) pair of the key tile starting at k0 is disallowed
// for some query of the tile (or lies beyond N): only such tiles evaluate the
// element mask.
__device__ __forceinline__ bool tile_is_edge(const TileRange& t, int k0, int N, int causal,
                                             int window) {
  return (k0 + kBN > N) || (causal && k0 + kBN - 1 > t.q0) ||
         (window >= 0 && (k0 < t.q_last - window || (!causal && k0 + kBN - 1 > t.q0 + window)));
}

// The band of the sliding-window page: keys i - w .. i + w, cut at j <= i when
// causal; window < 0 disables the band.
__device__ __forceinline__ bool key_allowed(int key, int qrow, int N, int causal, int window) {
  bool ok = key < N;
  if (causal) ok = ok && key <= qrow;
  if (window >= 0) ok = ok && key >= qrow - window && (causal || key <= qrow + window);
  return ok;
}

}  // namespace mi355attn
