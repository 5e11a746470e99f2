// Fused attention forward, E4M3 inputs with per-block descales, for gfx950.
//
// Same tiling, online softmax, masking and scheduling as the bf16 kernel
// (see attn_fwd_bf16.hip), with both contractions on the fp8 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4, fp32 accumulation): [JJ] section 2.3
// (the forward pass adapted to FP8 GEMMs) and [WGC] section 3 (per-block
// scaling, FP32 accumulation, BF16 output).
//
// Dequantisation is folded into scalars, never applied per element:
//  * a 128-row query tile is exactly one Q scaling block and a 64-key tile
//    lies inside one K/V scaling block, so the score scale of a tile is the
//    single number |scale| * log2(e) * dq * dk[block];
//  * P is converted to E4M3 as p * 2^8 (p <= 1, so p * 256 <= 256 < 448; the
//    power of two is exact) while the row sum l keeps the unrounded p;
//  * the output accumulator is kept in units of the current V block's descale:
//    when the V block changes, the online-softmax rescale factor also carries
//    dv_old / dv_new, and the epilogue multiplies by dv_last / (256 l).
// The V tile is stored in LDS with bits 2 and 3 of each key offset swapped, so
// that ds_read_b64_tr_b8 (8 consecutive LDS rows of one column per lane) hands
// every lane exactly the 32 keys whose probabilities it holds in registers.
#include "attn_device.h"
#include "attn_internal.h"

#include <type_traits>

namespace mi355attn {
namespace {

// 16-byte chunk swizzles for E4M3 tiles (rows of D bytes): K is read 16 B per
// lane from consecutive rows at one chunk; V is read by 16-lane groups as 8
// rows x one 16-byte chunk.
template <int D>
__device__ __forceinline__ int swz_k8(int r) {
  if constexpr (D == 128) return (r & 7) ^ ((r >> 3) & 1);
  else return (((r >> 2) & 1) << 1) | (((r >> 1) ^ (r >> 3)) & 1);
}
template <int D>
__device__ __forceinline__ int swz_v8(int r) {
  if constexpr (D == 128) return r & 7;
  else return (r >> 1) & 3;
}
// LDS row of key offset k within a tile: swap bits 2 and 3 (an involution).
__device__ __forceinline__ int v8_row(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

__device__ __forceinline__ int cvt4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

template <int D>
__global__ __launch_bounds__(kThreads, 2)
void attn_fwd_fp8_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
                         const uint8_t* __restrict__ V, uint16_t* __restrict__ O,
                         float* __restrict__ LSE, const float* __restrict__ DQ,
                         const float* __restrict__ DK, const float* __restrict__ DV, int N,
                         int nqt, float c0, int causal, int window, int qsign) {
  constexpr int DCH = D / 16;                  // 16-byte chunks per row
  constexpr int KSTEPS = D / 64;               // MFMA k-steps of QK^T
  constexpr int DBLK = D / 32;                 // 32-wide d blocks of O^T
  constexpr int TILE = kBN * D;                // bytes of one K or V tile
  constexpr int LOADS = kBN * DCH / kThreads;  // 16-byte loads per thread per tile
  constexpr float kPScale = 256.f;             // P is stored as E4M3(p * 2^8)
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];  // K0 K1 V0 V1
  lds_char* lds = (lds_char*)smem;

  const TileRange tr = tile_range(N, nqt, causal, window);
  const int bh = tr.bh, q0 = tr.q0, kt0 = tr.kt0, kt1 = tr.kt1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int qrow = q0 + wave * 32 + l32;
  const size_t head = (size_t)bh * N * D;
  const int nsb = (N + 127) / 128;             // scaling blocks per head
  const float* dk = DK + (size_t)bh * nsb;
  const float* dv = DV + (size_t)bh * nsb;
  const float cq = c0 * DQ[(size_t)bh * nsb + q0 / 128];

  // Q fragments: lane holds q8[qrow][64t + 32h .. +31].
  i32x8 qf[KSTEPS];
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t) {
    i32x4 x0 = {0, 0, 0, 0}, x1 = {0, 0, 0, 0};
    if (qrow < N) {
      const uint8_t* p = Q + head + (size_t)qrow * D + 64 * t + 32 * h;
      x0 = *(const i32x4*)p;
      x1 = *(const i32x4*)(p + 16);
    }
    x0 ^= qsign;
    x1 ^= qsign;
    qf[t] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  }

  i32x4 kst[LOADS], vst[LOADS];
  auto gload = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int chunk = tid + u * kThreads;
      const int row = chunk / DCH, col = chunk % DCH;
      const int key = kt * kBN + row;
      if (key < N) {
        const size_t off = head + (size_t)key * D + col * 16;
        kst[u] = *(const i32x4*)(K + off);
        vst[u] = *(const i32x4*)(V + off);
      } else {
        kst[u] = i32x4{0, 0, 0, 0};
        vst[u] = i32x4{0, 0, 0, 0};
      }
    }
  };
  auto sstore = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int chunk = tid + u * kThreads;
      const int row = chunk / DCH, col = chunk % DCH;
      *(lds_i32x4*)(lds + buf * TILE + row * D + ((col ^ swz_k8<D>(row)) << 4)) = kst[u];
      const int vr = v8_row(row);
      *(lds_i32x4*)(lds + (2 + buf) * TILE + vr * D + ((col ^ swz_v8<D>(vr)) << 4)) = vst[u];
    }
  };

  f32x16 oacc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) oacc[db] = f32x16{};
  float m = -INFINITY;                          // running max of c * s (base 2)
  float l = 0.f;                                // running sum (this lane's keys)
  float v_unit = kt0 < kt1 ? dv[(kt0 * kBN) / 128] : 1.f;  // descale O is kept in

  if (kt0 < kt1) {
    gload(kt0);
    sstore(0);
  }
  __syncthreads();

  // One key tile; only EDGE tiles carry mask code.
  auto step = [&](auto edge_tag, int kt) __attribute__((always_inline)) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const int buf = (kt - kt0) & 1;
    const bool more = kt + 1 < kt1;
    if (more) gload(kt + 1);
    const lds_char* Ks = lds + buf * TILE;
    const lds_char* Vs = lds + (2 + buf) * TILE;
    const int k0 = kt * kBN;
    const float c = cq * dk[k0 / 128];
    const float dv_t = dv[k0 / 128];

    // ---- S^T = K Q^T (fp8 x fp8 -> fp32)
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
      const int row = kb * 32 + l32;
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) {
        const int ch = 4 * t + 2 * h;
        const i32x4 a0 = *(const lds_i32x4*)(Ks + row * D + ((ch ^ swz_k8<D>(row)) << 4));
        const i32x4 a1 = *(const lds_i32x4*)(Ks + row * D + (((ch + 1) ^ swz_k8<D>(row)) << 4));
        const i32x8 kf = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf[t], sacc[kb], 0, 0, 0, 0,
                                                                   0, 0);
      }
    }

    // ---- online softmax (identical to the bf16 kernel, per-tile scale c)
    if constexpr (EDGE) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
          if (!key_allowed(key, qrow, N, causal, window)) sacc[kb][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    mx = halves_max(mx);
    const float mnew = fmaxf(m, mx == -INFINITY ? -INFINITY : mx * c);
    const float muse = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = fast_exp2(m - muse);

    // P as E4M3(p * 256), byte j of the B operand = key of sacc[j / 16][j % 16]
    i32x8 pf;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float s = sacc[kb][4 * w + e];
          p[e] = fast_exp2(fmaf(s, c, -muse));
          if constexpr (EDGE) p[e] = s == -INFINITY ? 0.f : p[e];
          rs += p[e];
        }
        pf[4 * kb + w] = cvt4(p[0] * kPScale, p[1] * kPScale, p[2] * kPScale, p[3] * kPScale);
      }
    l = l * alpha + rs;
    const float f = alpha * (v_unit / dv_t);   // also moves O into dv_t units
    if (__ballot(f != 1.f)) {
#pragma unroll
      for (int db = 0; db < DBLK; ++db) oacc[db] *= f;
    }
    v_unit = dv_t;
    m = mnew;

    // ---- O^T += V^T P^T: one K=64 MFMA per 32-wide d block. Lane (d, h)
    //      reads LDS rows 16t + 8h .. +7 of column d for t = 0..3.
    const int g = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const int col = db * 32 + 16 * (g & 1) + 8 * (sl & 1);   // this source lane's 8 bytes
      i32x8 va;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = 16 * t + 8 * (g >> 1) + (sl >> 1);
        const int a = r * D + (((col >> 4) ^ swz_v8<D>(r)) << 4) + (col & 15);
        const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(Vs + a));
        va[2 * t] = x[0];
        va[2 * t + 1] = x[1];
      }
      oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pf, oacc[db], 0, 0, 0, 0, 0, 0);
    }

    if (more) sstore(buf ^ 1);
    __syncthreads();
  };

  const InteriorSpan span = interior_span(tr, N, causal, window);
  int kt = kt0;
  for (; kt < span.ia; ++kt) step(std::true_type{}, kt);
  for (; kt < span.ib; ++kt) step(std::false_type{}, kt);
  for (; kt < kt1; ++kt) step(std::true_type{}, kt);

  // ---- epilogue: O = O_acc * dv_last / (256 l), LSE = ln 2 * (m + log2 l)
  const float lt = halves_sum(l);
  const float inv = lt > 0.f ? v_unit / (kPScale * lt) : 0.f;
  if (qrow < N) {
    uint16_t* orow = O + head + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(oacc[db][4 * g4 + e] * inv);
        *(bf16x4*)(orow + db * 32 + 8 * g4 + 4 * h) = o4;
      }
    if (h == 0) {
      const float muse = m == -INFINITY ? 0.f : m;
      LSE[(size_t)bh * N + qrow] = lt > 0.f ? (muse + log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_attn_fwd_fp8(const FwdArgs& a, hipStream_t stream) {
  const int nqt = (a.N + kBM - 1) / kBM;
  const int G = nqt * a.BH;  // bounded by the C ABI's shape checks
  const float c0 = fabsf(a.scale) * kLog2e;
  const int qsign = a.scale < 0.f ? (int)0x80808080u : 0;
  const uint8_t* q = (const uint8_t*)a.q;
  const uint8_t* k = (const uint8_t*)a.k;
  const uint8_t* v = (const uint8_t*)a.v;
  uint16_t* o = (uint16_t*)a.o;
  if (a.d == 128)
    hipLaunchKernelGGL(attn_fwd_fp8_kernel<128>, dim3(G), dim3(kThreads), 0, stream, q, k, v, o,
                       a.lse, a.dq, a.dk, a.dv, a.N, nqt, c0, a.causal, a.window, qsign);
  else
    hipLaunchKernelGGL(attn_fwd_fp8_kernel<64>, dim3(G), dim3(kThreads), 0, stream, q, k, v, o,
                       a.lse, a.dq, a.dk, a.dv, a.N, nqt, c0, a.causal, a.window, qsign);
  return hipGetLastError();
}

}  // namespace mi355attn
