// Device-side helpers shared by the bf16 and fp8 attention kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace mi355attn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
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

constexpr int kBM = 128;      // query rows of a 4-wave workgroup, 32 per wave
constexpr int kBN = 64;       // keys per K/V tile
constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994530942f;
// Word 3 of a raw buffer resource (no swizzle, 32-bit format field) for gfx950;
// out-of-range offsets read as zero.
constexpr int kRsrcWord3 = 0x00020000;
typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer descriptor (4 dwords: base, base high | stride 0, size in bytes,
// word 3) over `bytes` bytes at `base`; reads at or past the size return zero.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const unsigned long long a = (unsigned long long)base;
  return i32x4{(int)(uint32_t)a, (int)(uint32_t)((a >> 32) & 0xffff), (int)bytes, kRsrcWord3};
}
// 16-byte HBM -> LDS copy of one lane's chunk (buffer_load_dwordx4 ... lds):
// the wave's 64 chunks land contiguously at lds_base + 16 * lane, read from
// the descriptor's base + soffset + voffset. On gfx950 the buffer range check
// compares the whole offset, soffset + voffset, with the descriptor's size
// (measured: a descriptor sized to size - soffset zeroes every chunk at
// soffset + voffset >= size - soffset, and chunks past a head's end read as
// zero with NaN-filled memory right behind it). So the kernels put a tile's
// offset in soffset over a descriptor of the whole head, and a chunk at or
// past the head's end reads as zero and touches no memory.
// Issued from inline assembly, so the compiler does not track its LDS write:
// the callers order it with explicit vmcnt waits and barriers. (The compiler
// cannot tell that the transposing LDS reads of one tile never touch the tile
// still being copied, and would otherwise wait for every copy in flight
// before each of them.) M0 carries the LDS address.
__device__ __forceinline__ void copy_to_lds16(i32x4 rsrc, const lds_char* lds_base, int voffset,
                                              int soffset) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"((uint32_t)(uintptr_t)lds_base), "v"(voffset), "s"(rsrc), "s"(soffset)
               : "memory", "m0");
}
// The same 16-byte HBM -> LDS copy from a flat global address, marked
// nontemporal (streamed data: gfx950 accepts the nt bit on this form, not on
// the buffer form). There is no range check: callers use it only for rows
// they have shown to lie inside their allocation.
__device__ __forceinline__ void copy_to_lds16_nt(const void* gaddr, const lds_char* lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
               :
               : "s"((uint32_t)(uintptr_t)lds_base), "v"(gaddr)
               : "memory", "m0");
}
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem_upto() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 16-byte chunk swizzles of bf16 K and V tiles in LDS (rows of 2 D bytes).
// K is read 16 B per lane from 32 consecutive rows at one chunk column; V is
// read 8 B per lane as 4 consecutive rows x 32 bytes per 16-lane group by the
// transposing read. The XOR keeps both conflict-free for 32- and 64-bank LDS
// organisations.
// At D = 256 a row is 512 bytes, which maps onto the banks like a 256-byte
// row (bank = byte offset mod 256), so the D = 128 patterns carry over.
template <int D>
__device__ __forceinline__ int bf16_swz_k(int r) {
  if constexpr (D >= 128) return r & 15;
  else return ((r >> 1) & 7) ^ ((r & 1) << 2);
}
template <int D>
__device__ __forceinline__ int bf16_swz_v(int r) {
  if constexpr (D >= 128) {
    const int p = r & 3;
    return ((p << 1) + (p >> 1)) << 1;
  } else {
    return (r & 3) << 1;
  }
}

// Bijective remap of the hardware workgroup id so that ids dispatched to the
// same XCD (w % 8, round-robin dispatch) get consecutive logical ids, i.e. the
// query tiles of one head share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int w, int G) {
  const int q = G / kXcds, r = G % kXcds;
  const int x = w % kXcds, slot = w / kXcds;
  return x * q + min(x, r) + slot;
}

// max(a, b) as v_med3_f32(a, b, +inf). A two-input fmaxf makes the compiler
// quiet both inputs first (two extra v_max_f32 x, x, x when they come from
// an MFMA or a lane permute); the three-input forms need no such step.
__device__ __forceinline__ float max2(float a, float b) {
  return __builtin_amdgcn_fmed3f(a, b, INFINITY);
}
__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// v_permlane32_swap of a value with itself leaves, in every lane l, the pair
// {x[l % 32], x[l % 32 + 32]} (in some order): the two halves of one query row
// in the S^T accumulator layout.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max of an array as levels of v_max3_f32 (N - 1 comparisons in about
// (N - 1) / 2 instructions, short dependency chains).
template <int N>
__device__ __forceinline__ float tree_max(const float* x) {
  if constexpr (N == 1) {
    return x[0];
  } else if constexpr (N == 2) {
    return max2(x[0], x[1]);
  } else {
    constexpr int G = N / 3, R = N % 3, M = G + (R == 1 ? 1 : 0);
    float y[M];
#pragma unroll
    for (int i = 0; i < G; ++i) y[i] = max3(x[3 * i], x[3 * i + 1], x[3 * i + 2]);
    if constexpr (R == 2) y[G - 1] = max3(x[N - 2], x[N - 1], y[G - 1]);
    if constexpr (R == 1) y[G] = x[N - 1];
    return tree_max<M>(y);
  }
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
// Sum of 8 packed bf16 values (one bf16x8) into fp32 with v_dot2_f32_bf16
// against (1, 1): products are exact, the additions are fp32.
__device__ __forceinline__ float sum_bf16x8(bf16x8 v, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[0], v[1]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[2], v[3]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[4], v[5]}, one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[6], v[7]}, one, acc, false);
}

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Work item of one workgroup: (batch*head, query tile) and its key-tile range.
struct TileRange {
  int bh, q0, q_last, kt0, kt1;
};

// Query tile qt of (batch*head) bh. bm: query rows per workgroup, bn: keys
// per key tile.
__device__ __forceinline__ TileRange tile_range_at(int bh, int qt, int N, int causal, int window,
                                                   int bm, int bn) {
  TileRange t;
  t.bh = bh;
  t.q0 = qt * bm;
  t.q_last = min(N, t.q0 + bm) - 1;
  // allowed keys of the whole query tile: [k_lo, k_hi)
  const int k_lo = window >= 0 ? max(0, t.q0 - window) : 0;
  const int k_hi = causal ? t.q_last + 1 : (window >= 0 ? min(N, t.q_last + window + 1) : N);
  t.kt0 = k_lo / bn;
  t.kt1 = (k_hi + bn - 1) / bn;
  return t;
}

// One query tile per workgroup. Within a head, causal problems visit their
// heaviest (last) query tiles first. All others go in ascending order: under
// a band, the first key tiles of a query tile are the last ones of the tile
// before it, so a new workgroup finds them in L2.
__device__ __forceinline__ TileRange tile_range(int N, int nqt, int causal, int window,
                                                int bm = kBM, int bn = kBN) {
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = (causal && window < 0) ? nqt - 1 - logical % nqt : logical % nqt;
  return tile_range_at(logical / nqt, qt, N, causal, window, bm, bn);
}

// Causal pairing: workgroup u takes the query tiles nqt-1-p and p of one head
// (p = u mod ceil(nqt/2); one tile when they coincide), heavier first. Under
// a causal mask their key-tile counts add up to the same total for every p,
// so every workgroup carries the same work and no short workgroups are left
// for the end of the grid.
struct TilePair {
  int bh, first, second;   // second < 0: a single tile
};
__device__ __forceinline__ TilePair tile_pair(int nqt) {
  const int npair = (nqt + 1) >> 1;
  const int u = xcd_remap(blockIdx.x, gridDim.x);
  TilePair t;
  t.bh = u / npair;
  const int p = u % npair;
  t.first = nqt - 1 - p;
  t.second = p != t.first ? p : -1;
  return t;
}

// Wave-uniform values that are needed only between query tiles (base
// pointers) are parked in VGPRs, so that the SGPRs stay free for the tile
// loop: the empty asm hides the value from the compiler's
// uniformity analysis, so it is held per lane; uniform() reads it back into
// an SGPR where it is used. The asm is re-issued at every use so that the
// read-back cannot be hoisted out of the loop.
__device__ __forceinline__ int park(int x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ int uniform(int parked) {
  return __builtin_amdgcn_readfirstlane(park(parked));
}
// A pointer, parked when P (else held as is).
template <bool P>
struct ParkedPtr {
  int lo, hi;
  __device__ __forceinline__ explicit ParkedPtr(const void* p) {
    const unsigned long long a = (unsigned long long)p;
    lo = (int)(uint32_t)a;
    hi = (int)(uint32_t)(a >> 32);
    if constexpr (P) {
      lo = park(lo);
      hi = park(hi);
    }
  }
  // wave-uniform read-back
  template <class T>
  __device__ __forceinline__ T* get() const {
    if constexpr (P)
      return (T*)(((unsigned long long)(uint32_t)uniform(hi) << 32) | (uint32_t)uniform(lo));
    else
      return (T*)(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo);
  }
  // per-lane read-back (for per-lane addresses)
  template <class T>
  __device__ __forceinline__ T* lanes() const {
    return (T*)(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo);
  }
};

// Key tiles [ia, ib) inside [kt0, kt1) are "interior": every key of the tile is
// allowed for every query of the query tile, so they need no element mask.
// Tiles before ia and from ib on are "edge" tiles.
struct InteriorSpan {
  int ia, ib;
};
__device__ __forceinline__ InteriorSpan interior_span(const TileRange& t, int N, int causal,
                                                      int window, int bn = kBN) {
  const int lo_need = window >= 0 ? max(0, t.q_last - window) : 0;   // smallest key all rows allow
  int hi_need = N;                                                     // one past the largest
  if (causal) hi_need = min(hi_need, t.q0 + 1);
  else if (window >= 0) hi_need = min(hi_need, t.q0 + window + 1);
  InteriorSpan s;
  s.ia = min(max((lo_need + bn - 1) / bn, t.kt0), t.kt1);
  s.ib = min(max(hi_need / bn, s.ia), t.kt1);
  return s;
}

// The allowed keys of query i (the band of the sliding-window page, both ends
// inclusive): j < N; j <= i when causal; with a window w >= 0 also
// j >= i - w and, when not causal, j <= i + w. For every query this is one
// range [lo, hi], which the kernels' edge-tile masks compute once per lane.

}  // namespace mi355attn
