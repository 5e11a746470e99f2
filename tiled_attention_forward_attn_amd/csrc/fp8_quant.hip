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

__device__ __forceinline__ int cvt4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

__device__ __forceinline__ float sat(float y) { return fminf(fmaxf(y, -kE4M3Max), kE4M3Max); }

template <int D, int MODE>
__global__ __launch_bounds__(kThreads)
void fp8_quant_kernel(const uint16_t* __restrict__ X, uint8_t* __restrict__ X8,
                      float* __restrict__ descale, int N, int nb) {
  constexpr int DCH = D / 8;                       // 16-byte chunks per row
  constexpr int LOADS = kRows * DCH / kThreads;    // 8 at d = 128, 4 at d = 64
  __shared__ float red[kThreads / 64];

  const int blk = blockIdx.x;                      // (bh, rb) flattened
  const int bh = blk / nb, rb = blk % nb;
  const size_t head = (size_t)bh * N * D;
  const int tid = threadIdx.x;

  i32x4 x[LOADS];
  float amax = 0.f;
#pragma unroll
  for (int u = 0; u < LOADS; ++u) {
    const int chunk = tid + u * kThreads;
    const int row = rb * kRows + chunk / DCH, col = chunk % DCH;
    x[u] = i32x4{0, 0, 0, 0};
    if (row < N) x[u] = __builtin_nontemporal_load((const i32x4*)(X + head + (size_t)row * D + col * 8));
#pragma unroll
    for (int e = 0; e < 4; ++e)
      amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(x[u][e])), fabsf(bf16_hi(x[u][e]))));
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
    const int row = rb * kRows + chunk / DCH, col = chunk % DCH;
    if (row < N) {
      i32x2 out;
      out[0] = cvt4(sat(bf16_lo(x[u][0]) * r), sat(bf16_hi(x[u][0]) * r),
                    sat(bf16_lo(x[u][1]) * r), sat(bf16_hi(x[u][1]) * r));
      out[1] = cvt4(sat(bf16_lo(x[u][2]) * r), sat(bf16_hi(x[u][2]) * r),
                    sat(bf16_lo(x[u][3]) * r), sat(bf16_hi(x[u][3]) * r));
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

template <int D>
hipError_t launch_d(const uint16_t* x, uint8_t* x8, float* ds, int BH, int N, int per_tensor,
                    hipStream_t s) {
  const int nb = (N + kRows - 1) / kRows;
  const int G = BH * nb;  // bounded by the C ABI's shape checks
  if (!per_tensor) {
    hipLaunchKernelGGL((fp8_quant_kernel<D, kPerBlock>), dim3(G), dim3(kThreads), 0, s, x, x8, ds, N, nb);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((fp8_quant_kernel<D, kAmaxOnly>), dim3(G), dim3(kThreads), 0, s, x, x8, ds, N, nb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fp8_amax_broadcast_kernel, dim3(1), dim3(1024), 0, s, ds, G);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fp8_quant_kernel<D, kConvertFromSlot>), dim3(G), dim3(kThreads), 0, s, x, x8, ds, N, nb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8_quantize(const void* x, void* x8, float* descale, int BH, int N, int d,
                               int per_tensor, hipStream_t stream) {
  if (d == 128)
    return launch_d<128>((const uint16_t*)x, (uint8_t*)x8, descale, BH, N, per_tensor, stream);
  return launch_d<64>((const uint16_t*)x, (uint8_t*)x8, descale, BH, N, per_tensor, stream);
}

}  // namespace mi355attn
