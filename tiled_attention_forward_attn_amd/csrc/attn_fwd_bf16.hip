// Fused attention forward, bf16 inputs, for gfx950 (MI355X / CDNA4).
//
// One workgroup of 4 waves owns a 128-row query tile of one (batch, head) and
// streams the allowed key/value tiles (64 keys each) through LDS, double
// buffered, so tile j+1's global loads are in flight while tile j is being
// multiplied. Scores, probabilities and the output accumulator never leave
// registers; the N x N score matrix is never formed. This is the tiled,
// fused scheme of [WGC] sections 1-2 (QK^T -> softmax statistics -> PV with
// running max/sum and output rescale) and [YT] sections 1.2 and 2.1.1
// (softmax + mask + matmul fused; global tile -> shared-memory tile ->
// register tile), mapped onto CDNA4 rather than Hopper:
//
//  * Each wave computes S^T = K Q^T for its 32 queries with
//    v_mfma_f32_32x32x16_bf16. In the transposed product every lane holds 16
//    keys of ONE query, so a row's max and sum are in-lane reductions plus a
//    single v_permlane32_swap with the lane holding the other 16 keys.
//  * The probabilities come out of the accumulator already in the B-operand
//    layout of the second product O^T = V^T P^T: P never moves between lanes
//    and never touches LDS (the register hand-off of [WGC] section 1).
//  * The V^T operand is read from the row-major V tile with ds_read_b64_tr_b16,
//    gfx950's transposing LDS read (4 keys x 1 column per lane per read).
//  * K and V tiles are XOR-swizzled in LDS at 16-byte granularity so the
//    32 rows a wave reads at once fall into distinct banks.
//  * The online softmax works in base 2 with log2(e) folded into the scale
//    (v_exp_f32 computes 2^x). The reference max of a row only moves when the
//    row max exceeds it by more than 8 (so p <= 2^8, exact in fp32 and fine in
//    bf16); the O rescale is skipped unless some row of the wave moved.
//  * Fully masked key tiles are never visited (causal / sliding-window block
//    skipping, [YT] section 2.1.2); only tiles straddling a mask edge or the
//    ragged end of the sequence evaluate the element mask.
//  * Workgroup ids are remapped so that the query tiles of one head land on
//    one XCD (dispatch is round-robin over the 8 XCDs) and share K/V in that
//    XCD's L2; masked problems issue their heaviest query tiles first.
#include "attn_device.h"
#include "attn_internal.h"

#include <type_traits>

namespace mi355attn {
namespace {

// 16-byte chunk swizzles. K is read 16 B per lane from 32 consecutive rows at
// one chunk column; V is read 8 B per lane as 4 consecutive rows x 32 bytes per
// 16-lane group by the transposing read. The XOR keeps both conflict-free for
// 32- and 64-bank LDS organisations.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (D == 128) return r & 15;
  else return ((r >> 1) & 7) ^ ((r & 1) << 2);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  if constexpr (D == 128) {
    const int p = r & 3;
    return ((p << 1) + (p >> 1)) << 1;
  } else {
    return (r & 3) << 1;
  }
}

// Slack (base-2 units) by which a row max may exceed the reference max before
// the reference moves: probabilities reach at most 2^8, fine for bf16.
constexpr float kRescaleSlack = 8.f;

template <int D>
__global__ __launch_bounds__(kThreads, 2)
void attn_fwd_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                          const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                          float* __restrict__ LSE, int N, int nqt, float c, int causal,
                          int window, int qsign) {
  constexpr int DCH = D / 8;                   // 16-byte chunks per row
  constexpr int KSTEPS = D / 16;               // MFMA k-steps of QK^T
  constexpr int DBLK = D / 32;                 // 32-wide d blocks of O^T
  constexpr int TILE = kBN * D * 2;            // bytes of one K or V tile
  constexpr int LOADS = kBN * DCH / kThreads;  // 16-byte loads per thread per tile
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];  // K0 K1 V0 V1
  lds_char* lds = (lds_char*)smem;

  const TileRange tr = tile_range(N, nqt, causal, window);
  const int bh = tr.bh, q0 = tr.q0, kt0 = tr.kt0, kt1 = tr.kt1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int qrow = q0 + wave * 32 + l32;
  const size_t head = (size_t)bh * N * D;

  // Q fragments (B operand of S^T = K Q^T): lane holds q[qrow][16t + 8h .. +7].
  bf16x8 qf[KSTEPS];
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t) {
    i32x4 x = {0, 0, 0, 0};
    if (qrow < N) x = *(const i32x4*)(Q + head + (size_t)qrow * D + 16 * t + 8 * h);
    x ^= qsign;  // exact sign flip for negative scales
    qf[t] = __builtin_bit_cast(bf16x8, x);
  }

  i32x4 kst[LOADS], vst[LOADS];
  auto gload = [&](int kt) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int chunk = tid + u * kThreads;
      const int row = chunk / DCH, col = chunk % DCH;
      const int key = kt * kBN + row;
      if (key < N) {
        const size_t off = head + (size_t)key * D + col * 8;
        kst[u] = *(const i32x4*)(K + off);
        vst[u] = *(const i32x4*)(V + off);
      } else {
        kst[u] = i32x4{0, 0, 0, 0};
        vst[u] = i32x4{0, 0, 0, 0};
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int chunk = tid + u * kThreads;
      const int row = chunk / DCH, col = chunk % DCH;
      *(lds_i32x4*)(lds + buf * TILE + row * D * 2 + ((col ^ swz_k<D>(row)) << 4)) = kst[u];
      *(lds_i32x4*)(lds + (2 + buf) * TILE + row * D * 2 + ((col ^ swz_v<D>(row)) << 4)) = vst[u];
    }
  };

  f32x16 oacc[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) oacc[db] = f32x16{};
  float m = -INFINITY;  // running max of c * s (base-2 units)
  float l = 0.f;        // running sum over this lane's 32 keys of each tile

  if (kt0 < kt1) {
    gload(kt0);
    sstore(0);
  }
  __syncthreads();

  // One key tile. EDGE tiles evaluate the element mask; interior tiles carry
  // no mask code at all (the compiler would otherwise if-convert the mask
  // into every tile).
  auto step = [&](auto edge_tag, int kt) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const int buf = (kt - kt0) & 1;
    const bool more = kt + 1 < kt1;
    if (more) gload(kt + 1);
    const lds_char* Ks = lds + buf * TILE;
    const lds_char* Vs = lds + (2 + buf) * TILE;

    // ---- S^T = K Q^T for 64 keys x this wave's 32 queries
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
      const int row = kb * 32 + l32;
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) {
        const int ch = 2 * t + h;
        const bf16x8 kf = *(const lds_bf16x8*)(Ks + row * D * 2 + ((ch ^ swz_k<D>(row)) << 4));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], sacc[kb], 0, 0, 0);
      }
    }

    // ---- online softmax. sacc[kb][i] is the score of key
    //      k0 + 32 kb + 8 (i/4) + 4 h + i%4 against query qrow.
    const int k0 = kt * kBN;
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
    const float mxs = mx == -INFINITY ? -INFINITY : mx * c;
    // The reference max only moves when a row max exceeds it by more than
    // kRescaleSlack (base 2), so p <= 2^kRescaleSlack and the O rescale is
    // rare; the final O / l and LSE are unchanged mathematically.
    const bool grow = mxs > m + kRescaleSlack;
    const float mnew = grow ? mxs : m;
    const float muse = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = fast_exp2(m - muse);

    bf16x8 pf[4];
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = fast_exp2(fmaf(sacc[kb][i], c, -muse));
        if constexpr (EDGE) p = sacc[kb][i] == -INFINITY ? 0.f : p;
        rs += p;
        pf[kb * 2 + (i >> 3)][i & 7] = (__bf16)p;
      }
    if (__ballot(grow)) {
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) oacc[db] *= alpha;
    }
    l += rs;
    m = mnew;

    // ---- O^T += V^T P^T. MFMA step s covers keys 16 s .. 16 s + 15 of the
    //      tile; lane (d, h) needs V at keys 16s + 4h + {0..3} and + 8.
    const int g = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r1 = 16 * s + 4 * (g >> 1) + (sl >> 2);
      const int r2 = r1 + 8;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const int col = db * 32 + 16 * (g & 1) + 4 * (sl & 3);
        const int a1 = r1 * D * 2 + (((col >> 3) ^ swz_v<D>(r1)) << 4) + ((col >> 2) & 1) * 8;
        const int a2 = r2 * D * 2 + (((col >> 3) ^ swz_v<D>(r2)) << 4) + ((col >> 2) & 1) * 8;
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Vs + a1));
        const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Vs + a2));
        const bf16x8 va = __builtin_bit_cast(
            bf16x8, i16x8{v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]});
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[s], oacc[db], 0, 0, 0);
      }
    }

    if (more) sstore(buf ^ 1);
    __syncthreads();
  };

  const InteriorSpan span = interior_span(tr, N, causal, window);
  int kt = kt0;
  for (; kt < span.ia; ++kt) step(std::true_type{}, kt);
  for (; kt < span.ib; ++kt) step(std::false_type{}, kt);
  for (; kt < kt1; ++kt) step(std::true_type{}, kt);

  // ---- epilogue: O = O^T / l (bf16, RNE), LSE = ln 2 * (m + log2 l)
  const float lt = halves_sum(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
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

hipError_t launch_attn_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  const int nqt = (a.N + kBM - 1) / kBM;
  const int G = nqt * a.BH;  // bounded by the C ABI's shape checks
  const float c = fabsf(a.scale) * kLog2e;  // |scale| * log2(e)
  const int qsign = a.scale < 0.f ? (int)0x80008000u : 0;
  const uint16_t* q = (const uint16_t*)a.q;
  const uint16_t* k = (const uint16_t*)a.k;
  const uint16_t* v = (const uint16_t*)a.v;
  uint16_t* o = (uint16_t*)a.o;
  if (a.d == 128)
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<128>, dim3(G), dim3(kThreads), 0, stream, q, k, v, o,
                       a.lse, a.N, nqt, c, a.causal, a.window, qsign);
  else
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<64>, dim3(G), dim3(kThreads), 0, stream, q, k, v, o,
                       a.lse, a.N, nqt, c, a.causal, a.window, qsign);
  return hipGetLastError();
}

}  // namespace mi355attn
