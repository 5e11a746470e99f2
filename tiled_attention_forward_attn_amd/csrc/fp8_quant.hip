// bf16 -> E4M3 quantisation with one scaling factor per 128-row block, gfx950.
//
// Dynamic per-block scaling into the E4M3 range whose maximum is 448 ([WGC]
// section 3; format of [JJ] section 1.5). Per block of 128 rows x d of one
// (batch, head):
//   amax = max |x|, r = fp32(448 / amax), descale = fp32(amax / 448)
//   code = E4M3(fp32(x * r)), round to nearest even, saturating at +-448
//   (amax == 0: r = 1, descale = 1; 0 < amax < 448 * 2^-126, where amax / 448
//   would not be a normal fp32 and 448 / amax could overflow: r = 2^126,
//   descale = 2^-126, its exact reciprocal, so every |x * r| < 448 and a
//   zero encodes as 0)
// The divisions are IEEE correctly rounded (the library is built without
// fast-math), the product is one fp32 multiply, and the conversion is
// v_cvt_pk_fp8_f32 (round to nearest even, OCP E4M3FN on gfx950) after a clamp
// to +-448, which makes it saturating.
//
// The kernel is HBM-bound: each workgroup reads its block once (32 KiB at
// d = 128) into registers with 16-byte coalesced loads, reduces the amax
// across the workgroup, and writes 8 bytes of codes per 16 bytes read; both
// carry the nontemporal hint (streamed data, touched once).
// Per-tensor mode (the naive baseline) needs a global amax first; it runs
//   1. the same kernel in "amax only" mode, each block writing its amax into
//      its own descale slot,
//   2. a one-workgroup reduction of all slots that writes the global amax
//      back into every slot,
//   3. the kernel in "convert" mode, each block reading the global amax from
//      its own slot and overwriting that slot with the descale,
// so no workspace, atomic or memset is needed and no slot is read after
// another block has overwritten it.
//
// Rotated mode (incoherent processing, [JJ] introduction and section 3: the
// page pairs FP8 block quantisation with it): every row x is replaced, before
// the block's amax and conversion, by its rotation x diag(s) H / sqrt(d) (H
// the Sylvester Hadamard matrix, s the caller's random signs). Applied with
// the same signs to Q and K it leaves Q K^T unchanged while spreading
// channels that are large in both over all d channels. Computed in fp32 in a
// fixed order, since these values decide the codes: sign flips (exact); the
// fast Walsh-Hadamard butterfly with stages h = 1, 2, ..., d/2, each output
// one rounded fp32 sum (j with bit h clear: x[j] + x[j+h]) or difference
// (x[j] - x[j+h]); one multiply by fp32(1/sqrt(d)). A row's d / 8 chunks of
// 8 values sit in d / 8 consecutive lanes (at most one 16-lane DPP row), so
// stages 1, 2, 4 are in-lane and stage 8 m (m = 1, 2, ...) pairs lane l with
// lane l ^ m through DPP moves, with no LDS traffic.
#include "attn_internal.h"

#include <math.h>

namespace mi355attn {
namespace {

typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;

constexpr int kRows = 128;  // rows per scaling block
constexpr int kThreads = 256;
constexpr float kE4M3Max = 448.0f;
constexpr float kAmaxMinNormal = 0x1.cp-118f;   // 448 * 2^-126 = 7 * 2^-120
constexpr float kMinNormal = 0x1p-126f;
constexpr float kMinNormalInv = 0x1p126f;

enum Mode { kPerBlock = 0, kAmaxOnly = 1, kConvertFromSlot = 2 };

__device__ __forceinline__ float bf16_lo(int w) { return __int_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(int w) { return __int_as_float(w & (int)0xffff0000u); }

__device__ __forceinline__ float block_max(float v, float* red) {
  // |x| >= 0, so a max over the float bit patterns as unsigned is exact.
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
  return r;
}

// Four E4M3 codes in one word. Each v_cvt_pk_fp8_f32 writes one half of its
// destination and keeps the other; the second conversion overwrites the half
// the first one keeps, so the first one's "old" value is a don't-care: a's
// own bits (a register that dies here) rather than a zero, which would cost a
// v_mov per word.
__device__ __forceinline__ int cvt4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

__device__ __forceinline__ float sat(float y) { return fminf(fmaxf(y, -kE4M3Max), kE4M3Max); }

// fp32(1 / sqrt(d)): the rotation's normalisation.
template <int D>
constexpr float inv_sqrt_d() { return D == 128 ? 0.08838834764831845f : 0.125f; }

// The 8 values of one chunk as fp32 (bf16 bits, exact).
__device__ __forceinline__ void unpack8(i32x4 w, float (&v)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = bf16_lo(w[e]);
    v[2 * e + 1] = bf16_hi(w[e]);
  }
}

// Value of lane l ^ M (M = 1, 2, 4, 8) by DPP moves within the 16-lane row:
// quad_perm [1,0,3,2] and [2,3,0,1] are l ^ 1 and l ^ 2; row_half_mirror is
// l ^ 7 and row_mirror l ^ 15, so l ^ 4 = (l ^ 7) ^ 3 and l ^ 8 = (l ^ 15) ^ 7.
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  int x = __float_as_int(v);
  if constexpr (M == 1) {
    x = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);
  } else if constexpr (M == 2) {
    x = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);
  } else if constexpr (M == 4) {
    x = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);   // row_half_mirror
    x = __builtin_amdgcn_mov_dpp(x, 0x1B, 0xF, 0xF, false);    // quad_perm [3,2,1,0]
  } else {
    static_assert(M == 8, "within a 16-lane row");
    x = __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false);   // row_mirror
    x = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);   // row_half_mirror
  }
  return __int_as_float(x);
}

// Butterfly stage h = 8 M across lanes col and col ^ M, for all LOADS
// chunks: the lane holding x[j] (bit M of col clear) keeps x[j] + x[j + h],
// its partner x[j] - x[j + h]. Both are fma(s, own, partner) with s = +-1: the
// product is exact and the one rounding is that of the sum or difference.
template <int M, int LOADS>
__device__ __forceinline__ void cross_all(float (&v)[LOADS][8], int col) {
  const float s = (col & M) ? -1.f : 1.f;
#pragma unroll
  for (int u = 0; u < LOADS; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) v[u][e] = fmaf(s, v[u][e], lane_xor<M>(v[u][e]));
}

// Rotation of the LOADS rows this lane holds chunk `col` of (see the header):
// sign flips from the lane's sign mask bits, in-lane butterfly stages 1, 2, 4,
// cross-lane stages 8 .. D/2 (lane ^ m), then the normalisation. Each stage
// runs over all chunks before the next, so a DPP move finds other chunks'
// work between it and the instruction that produced its source (the
// shuffle-based form, one chunk at a time, took 336 us for a B16 H16 N8192
// d128 tensor; this one 141 us, bit-identical).
template <int D, int LOADS>
__device__ __forceinline__ void rotate_all(float (&v)[LOADS][8], int col, uint32_t sign_bits) {
#pragma unroll
  for (int u = 0; u < LOADS; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      v[u][e] = __uint_as_float(__float_as_uint(v[u][e]) ^ (((sign_bits >> e) & 1u) << 31));
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int u = 0; u < LOADS; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (!(e & h)) {
          const float a = v[u][e], b = v[u][e + h];
          v[u][e] = a + b;
          v[u][e + h] = a - b;
        }
  cross_all<1>(v, col);
  cross_all<2>(v, col);
  cross_all<4>(v, col);
  if constexpr (D / 8 > 8) cross_all<8>(v, col);
#pragma unroll
  for (int u = 0; u < LOADS; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) v[u][e] = v[u][e] * inv_sqrt_d<D>();
}

// ROT: rotate every row first (see the header); `signs` holds the d signs
// (a byte < 0 means -1). Without ROT, signs is unused.
template <int D, int MODE, bool ROT>
__global__ __launch_bounds__(kThreads)
void fp8_quant_kernel(const uint16_t* __restrict__ X, uint8_t* __restrict__ X8,
                      float* __restrict__ descale, const int8_t* __restrict__ signs, int N, int nb) {
  constexpr int DCH = D / 8;                       // 16-byte chunks per row
  constexpr int LOADS = kRows * DCH / kThreads;    // 8 at d = 128, 4 at d = 64
  static_assert(kThreads % DCH == 0, "a lane keeps its column in every round");
  __shared__ float red[kThreads / 64];

  const int blk = blockIdx.x;                      // (bh, rb) flattened
  const int bh = blk / nb, rb = blk % nb;
  const size_t head = (size_t)bh * N * D;
  const int tid = threadIdx.x;
  const int col = tid % DCH;                       // this lane's chunk of every row it holds

  uint32_t sign_bits = 0;
  if constexpr (ROT) {
    const i32x2 sw = *(const i32x2*)(signs + col * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      sign_bits |= (uint32_t)((((e < 4 ? sw[0] : sw[1]) >> (8 * (e & 3) + 7)) & 1)) << e;
  }

  // the block's values: packed bf16 as loaded, or (ROT) the rotated fp32
  i32x4 x[ROT ? 1 : LOADS];
  float v[ROT ? LOADS : 1][8];
  float amax = 0.f;
#pragma unroll
  for (int u = 0; u < LOADS; ++u) {
    const int chunk = tid + u * kThreads;
    const int row = rb * kRows + chunk / DCH;
    i32x4 w = {0, 0, 0, 0};
    if (row < N) w = __builtin_nontemporal_load((const i32x4*)(X + head + (size_t)row * D + col * 8));
    if constexpr (ROT) {
      unpack8(w, v[u]);   // rows past N are zero, and so is their rotation
    } else {
      x[u] = w;
      float f[8];
      unpack8(w, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(f[e]));
    }
  }
  if constexpr (ROT) {
    rotate_all<D, LOADS>(v, col, sign_bits);
#pragma unroll
    for (int u = 0; u < LOADS; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[u][e]));
  }

  if constexpr (MODE == kConvertFromSlot) {
    amax = descale[blk];
  } else {
    amax = block_max(amax, red);
    if constexpr (MODE == kAmaxOnly) {
      if (tid == 0) descale[blk] = amax;
      return;
    }
  }

  const bool tiny = amax < kAmaxMinNormal;   // includes amax == 0
  const float r = amax == 0.f ? 1.f : (tiny ? kMinNormalInv : kE4M3Max / amax);
#pragma unroll
  for (int u = 0; u < LOADS; ++u) {
    const int chunk = tid + u * kThreads;
    const int row = rb * kRows + chunk / DCH;
    if (row < N) {
      float f[8];
      if constexpr (ROT) {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = v[u][e];
      } else {
        unpack8(x[u], f);
      }
      i32x2 out;
      out[0] = cvt4(sat(f[0] * r), sat(f[1] * r), sat(f[2] * r), sat(f[3] * r));
      out[1] = cvt4(sat(f[4] * r), sat(f[5] * r), sat(f[6] * r), sat(f[7] * r));
      __builtin_nontemporal_store(out, (i32x2*)(X8 + head + (size_t)row * D + col * 8));
    }
  }
  if (tid == 0) descale[blk] = amax == 0.f ? 1.f : (tiny ? kMinNormal : amax / kE4M3Max);
}

// One workgroup: global max over all slots, written back into every slot.
__global__ __launch_bounds__(1024)
void fp8_amax_broadcast_kernel(float* __restrict__ slots, int n) {
  __shared__ float red[16];
  float v = 0.f;
  for (int i = threadIdx.x; i < n; i += 1024) v = fmaxf(v, slots[i]);
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float g = red[0];
  for (int i = 1; i < 16; ++i) g = fmaxf(g, red[i]);
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += 1024) slots[i] = g;
}

template <int D, bool ROT>
hipError_t launch_d(const uint16_t* x, uint8_t* x8, float* ds, const int8_t* signs, int BH, int N,
                    int per_tensor, hipStream_t s) {
  const int nb = (N + kRows - 1) / kRows;
  const int G = BH * nb;  // bounded by the C ABI's shape checks
  if (!per_tensor) {
    hipLaunchKernelGGL((fp8_quant_kernel<D, kPerBlock, ROT>), dim3(G), dim3(kThreads), 0, s, x, x8, ds,
                       signs, N, nb);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((fp8_quant_kernel<D, kAmaxOnly, ROT>), dim3(G), dim3(kThreads), 0, s, x, x8, ds,
                     signs, N, nb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fp8_amax_broadcast_kernel, dim3(1), dim3(1024), 0, s, ds, G);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fp8_quant_kernel<D, kConvertFromSlot, ROT>), dim3(G), dim3(kThreads), 0, s, x, x8,
                     ds, signs, N, nb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8_quantize(const void* x, void* x8, float* descale, const int8_t* signs, int BH,
                               int N, int d, int per_tensor, hipStream_t stream) {
  const uint16_t* xb = (const uint16_t*)x;
  uint8_t* q = (uint8_t*)x8;
  if (signs) {
    if (d == 128) return launch_d<128, true>(xb, q, descale, signs, BH, N, per_tensor, stream);
    return launch_d<64, true>(xb, q, descale, signs, BH, N, per_tensor, stream);
  }
  if (d == 128) return launch_d<128, false>(xb, q, descale, nullptr, BH, N, per_tensor, stream);
  return launch_d<64, false>(xb, q, descale, nullptr, BH, N, per_tensor, stream);
}

}  // namespace mi355attn
