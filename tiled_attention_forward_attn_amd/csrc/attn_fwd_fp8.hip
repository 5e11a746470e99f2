// Fused attention forward, E4M3 inputs with per-block descales, for gfx950.
//
// Same tiling, pipeline, masking and scheduling as the bf16 kernel (see
// attn_fwd_bf16.hip), with both contractions on the fp8 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4, fp32 accumulation): [JJ] section 2.3
// (the forward pass adapted to FP8 GEMMs) and [WGC] section 3 (per-block
// scaling, FP32 accumulation, BF16 output).
//
// Dequantisation is folded into scalars, never applied per element:
//  * a 128-row query tile is exactly one Q scaling block and a 64- or
//    128-key tile lies inside one K/V scaling block, so the score scale of a
//    tile is the single number |scale| * log2(e) * dq * dk[block];
//  * a tile's V descale never rescales O. It is split as dv_t = f_t * 2^e_t
//    with f_t in [1/2, 1): the mantissa enters P, stored as
//    E4M3(p * f_t * 2^8) (2^8 and log2 f_t folded into the exp argument),
//    and 2^e_t is the E8M0 A-operand scale of the PV MFMA (one byte, the
//    same in every lane), so P keeps the same precision floor whatever the
//    block descales are, and a zero descale (scale byte 0, 2^-127) still
//    leaves P for the row sum;
//  * the running max m of each row (log2 units) is kept as an integer, the
//    ceiling of the exact running max, so p <= 1. Its growth is never
//    applied to O by multiplication: O and l stay in units of a reference
//    m_ref (the row's first finite m), and tile t's PV product is scaled by
//    2^(m_t - m_ref) through the E8M0 B-operand scale of
//    v_mfma_scale_f32_32x32x64_f8f6f4 (one byte per lane, the lane's own
//    query). Only when m_t - m_ref would exceed kMaxShift are O and l
//    rebased, by an exact power of two. The online softmax of [WGC] section
//    2 is unchanged in value: every tile's weights still relate to the
//    running max; only where its rescale is applied moves;
//  * the row sum l is the sum of the stored E4M3 weights, the values that
//    multiply V, so the normalised weights add up to one and the rounding of
//    the largest weight largely cancels. Each tile's sum is taken on the
//    matrix core (one v_mfma_scale_f32_16x16x128_f8f6f4 of P^T, the PV B
//    operand, against a constant 0/1 A operand chosen so that each lane
//    receives the sum for the query it owns, see ones_operand), then added in
//    fp32 with the factor 2^(m_t - m_ref) / f_t.
// A second instance (QBF) keeps Q and K in bf16 and computes S = Q K^T on the
// bf16 matrix cores, with only V and P in E4M3: the score error that E4M3 Q
// and K carry on data with large, aligned outlier channels (it grows with
// |s|) is gone, while PV keeps the fp8 contraction. Everything from the
// scores on is shared with the all-E4M3 instance.
// The V tile is stored in LDS with bits 2 and 3 of each key offset swapped, so
// that ds_read_b64_tr_b8 (8 consecutive LDS rows of one column per lane) hands
// every lane exactly the 32 keys whose probabilities it holds in registers.
#include <type_traits>

#include "attn_device.h"
#include "attn_internal.h"

namespace mi355attn {
namespace {

// Keys per tile; each size divides the 128-row scaling block. E4M3 takes
// 128-key tiles (half the per-tile softmax and barrier work per key); the
// bf16-score instance keeps 64, where 128 would not fit the registers.
template <int D, bool QBF>
constexpr int fp8_bn() { return !QBF ? 128 : 64; }
constexpr float kPScaleLog2 = 8.f;     // P is stored as E4M3(p * f * 2^8)
constexpr float kMaxShift = 64.f;      // largest m - m_ref applied through the MFMA scale
constexpr int kE8M0One = 127;          // E8M0 scale byte of 1.0

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

// A operand of the row-sum MFMA. In v_mfma_*_16x16x128_f8f6f4 lane l holds
// A row l % 16 over k chunk c = l / 16 (32 k values), and B column l % 16 over
// the same chunk. Taking P's operand as B, chunk c of column n is the 32 keys
// of lane n + 16c, i.e. query n + 16 (c % 2), key half c / 2. Row r of A is
// one on the chunks with c % 2 == (r / 4) % 2 and zero elsewhere, so
// D[r][n] = l(query n + 16 ((r / 4) % 2)). Lane l receives rows 4 (l / 16) ..
// +3 of column l % 16: the sum of query l % 32, its own, in all four values.
// Every byte of a lane's A operand holds the same value, and A and B are both
// E4M3, so the pairing does not depend on how the instruction orders k within
// a lane: byte b of A's lane r + 16c always meets byte b of B's lane n + 16c.
// (An FP4 A operand would need half the registers, but its k order within a
// lane is not the E4M3 one, and a lane-constant A then mixes the two queries.)
__device__ __forceinline__ i32x8 ones_operand(int lane) {
  const int one4 = ((lane >> 4) & 1) == ((lane >> 2) & 1) ? 0x38383838 : 0;  // 4 x E4M3 1.0
  return i32x8{one4, one4, one4, one4, one4, one4, one4, one4};
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

// QBF: Q and K are bf16 and S = Q K^T runs on bf16 MFMAs; otherwise all E4M3.
template <int D, bool QBF>
struct Fp8Fwd {
  using QKFrag = std::conditional_t<QBF, bf16x8, i32x8>;
  static constexpr int BN = fp8_bn<D, QBF>();
  static constexpr int NH = BN / 64;                         // 64-key halves (one PV MFMA k-step)
  static constexpr int KSTEPS = QBF ? D / 16 : D / 64;      // MFMA k-steps of QK^T
  static constexpr int DBLK = D / 32;                       // 32-wide d blocks of O^T
  static constexpr int NKB = BN / 32;                       // 32-key blocks of S^T
  static constexpr int KBYTES = QBF ? 2 : 1;                // bytes per Q / K element
  static constexpr int KDCH = D * KBYTES / 16;              // 16-byte chunks per K row
  static constexpr int VDCH = D / 16;                       // 16-byte chunks per V row
  static constexpr int KTILE = BN * D * KBYTES;             // bytes of one K tile
  static constexpr int VTILE = BN * D;                      // bytes of one V tile
  static constexpr int KLOADS = KTILE / (16 * kThreads);    // 16-byte copies per thread
  static constexpr int VLOADS = VTILE / (16 * kThreads);
  // Copy round u of a tile lands kThreads / KDCH (or / VDCH) rows below round
  // 0. Both swizzles depend on row bits 0..3 only and the V key order swaps
  // bits 2 and 3, so round u's LDS offset is round 0's plus u * 16 * kThreads:
  // one offset register per tensor, the rest in the scalar offset.
  static_assert((kThreads / KDCH) % 16 == 0 && (kThreads / VDCH) % 16 == 0, "copy rounds");

  lds_char* kl[2];
  lds_char* vl[2];
  int N, causal, window, kt0, kt1, qrow;
  int lane, wave, h, l32;
  i32x4 kres, vres;
  int koff, voff;     // LDS byte offset of this lane's copy in round 0
  int krow, kswz;     // E4M3 K reads: l32 * D and swz_k8(l32) << 4
  const float* dk;
  const float* dv;
  float cq;
  // state
  QKFrag qf[KSTEPS];
  f32x16 oacc[DBLK];
  float l;            // row sum, units of 2^(m_ref - 8) (both key halves)
  i32x8 ones;
  f32x16 sacc[NKB];
  i32x8 pbuf[2][NH];
  QKFrag kf[NKB][KSTEPS];
  i32x8 vf[DBLK];
  float m;           // running max (log2 units), an integer or -inf
  float m_ref;       // units of O and l (log2), -inf until m is finite
  int sa[2];         // E8M0 byte of 2^e_t (V descale exponent) for P set 0 / 1
  int sb[2];         // E8M0 byte of 2^(m_t - m_ref) for P set 0 / 1
  float lf[2];       // 2^(m_t - m_ref) / f_t for P set 0 / 1

  template <int ST>
  __device__ __forceinline__ void issue_k(int kt) {
#pragma unroll
    for (int u = 0; u < KLOADS; ++u)
      copy_to_lds16(kres, kl[ST] + (u * 4 + wave) * 1024, koff,
                    (int)((uint32_t)kt * KTILE + u * 16 * kThreads));
  }
  template <int ST>
  __device__ __forceinline__ void issue_v(int kt) {
#pragma unroll
    for (int u = 0; u < VLOADS; ++u)
      copy_to_lds16(vres, vl[ST] + (u * 4 + wave) * 1024, voff,
                    (int)((uint32_t)kt * VTILE + u * 16 * kThreads));
  }

  // A operand of O^T += V^T P^T for the 64-key half hh: lane (d, h) reads LDS
  // rows 64 hh + 16t + 8h .. +7 of column d for t = 0..3 (the swapped key
  // order makes these its P's keys).
  template <int ST>
  __device__ __forceinline__ void read_v(int hh) {
    const lds_char* Vs = vl[ST];
    const int g = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const int col = db * 32 + 16 * (g & 1) + 8 * (sl & 1);  // this source lane's 8 bytes
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = 64 * hh + 16 * t + 8 * (g >> 1) + (sl >> 1);
        const int a = r * D + (((col >> 4) ^ swz_v8<D>(r)) << 4) + (col & 15);
        const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(Vs + a));
        vf[db][2 * t] = x[0];
        vf[db][2 * t + 1] = x[1];
      }
    }
  }

  // K fragments (A operand of S^T = K Q^T for 32-key block kb) and S^T of
  // the whole tile. The blocks' accumulator chains advance together, k-step
  // by k-step, and scheduling groups (0x100 = LDS reads, 0x008 = MFMAs) keep
  // the fragment reads a fixed distance ahead of the MFMAs that use them;
  // left to itself the compiler streams a block through one register set and
  // each MFMA waits a whole LDS round trip. The groups take the LDS reads that
  // precede them, so the caller issues its V reads after this function.
  // bf16 K: lane holds K[32 kb + l32][16 t + 8 h .. +7].
  // E4M3 K: lane holds K8[32 kb + l32][64 t + 32 h .. +31], chunks 4t + 2h
  // and 4t + 2h + 1 of its row. Rows 32 kb + l32 share the swizzle of l32 (it
  // reads row bits 0..3), so block kb is a constant offset. The four chunk
  // addresses are rebuilt every tile from two registers (one v_bitop3 each:
  // krow has no bits where the chunk index sits) rather than kept live across
  // the loop, where they would be spilled; the empty asm stops the compiler
  // from hoisting them.
  template <int ST>
  __device__ __forceinline__ void read_k_qk() {
    static_assert(!QBF || NKB == 2, "bf16-score tiles hold two 32-key blocks");
    int ko[KSTEPS][2] = {};
    if constexpr (!QBF) {
      int sw = kswz;
      asm volatile("" : "+v"(sw));
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) {
        const int ch = 4 * t + 2 * h;
        ko[t][0] = krow | ((ch << 4) ^ sw);
        ko[t][1] = krow | (((ch + 1) << 4) ^ sw);
      }
    }
    if constexpr (QBF) {
      // each step's two fragments read three steps ahead (+1.1% at B16 H16
      // N8192 in a same-box A/B, bit-identical)
      bf16x8 f[KSTEPS][NKB];
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int row = kb * 32 + l32;
          const int ch = 2 * t + h;
          f[t][kb] = *(const lds_bf16x8*)(kl[ST] + row * D * 2 + ((ch ^ bf16_swz_k<D>(row)) << 4));
        }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[t][kb], qf[t], sacc[kb], 0, 0, 0);
      constexpr int kKAhead = 3;
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kKAhead, 0);
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        if (t + kKAhead < KSTEPS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    } else {
      // each fragment (two 16-byte reads) read kE8Ahead MFMAs ahead
      // (same-box A/B, bit-identical: +1.6 .. 2.1% at d = 128 with one MFMA
      // ahead, +1% at d = 64 with two)
      constexpr int kE8Ahead = D == 64 ? 2 : 1;
      i32x8 f[KSTEPS][NKB];
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const i32x4 a0 = *(const lds_i32x4*)(kl[ST] + kb * 32 * D + ko[t][0]);
          const i32x4 a1 = *(const lds_i32x4*)(kl[ST] + kb * 32 * D + ko[t][1]);
          f[t][kb] = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f[t][kb], qf[t], sacc[kb], 0, 0,
                                                                     0, 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kE8Ahead, 0);
#pragma unroll
      for (int i = 0; i < KSTEPS * NKB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i + kE8Ahead < KSTEPS * NKB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
  }

  template <int PB>
  __device__ __forceinline__ void pv(int hh) {
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
      oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[db], pbuf[PB][hh], oacc[db], 0, 0,
                                                                 0, sa[PB], 0, sb[PB]);
    const f32x4 rs = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, pbuf[PB][hh], f32x4{}, 0,
                                                                      0, 0, 0, 0, 0);
    l = fmaf(rs[0], lf[PB], l);
  }
  // PV of P set PB, V stage PB: halves after the first read their V
  // fragments here (the first half's are read ahead by the caller)
  template <int PB>
  __device__ __forceinline__ void pv_rest() {
    pv<PB>(0);
#pragma unroll
    for (int hh = 1; hh < NH; ++hh) {
      read_v<PB>(hh);
      pv<PB>(hh);
    }
  }

  // Online softmax of S(kt) into P set PB (E4M3 of p * f * 2^8; byte j of
  // half hh's operand is the key of sacc[2 hh + j / 16][j % 16]).
  template <bool EDGE, int PB>
  __device__ __forceinline__ void softmax(int kt) {
    const int k0 = kt * BN;
    const float c = QBF ? cq : cq * dk[k0 / 128];   // bf16 scores carry no descale
    // V descale of the tile = f * 2^(e): f in [1/2, 1) into P, 2^e into the
    // PV A scale (E8M0 bytes 1 .. 254 cover every normal descale; zero and
    // subnormal descales get byte 0, 2^-127, and f = 1/2)
    const float dvt = dv[k0 / 128];
    const int dexp = __builtin_amdgcn_frexp_expf(dvt);
    const bool dnorm = dvt >= 1.17549435e-38f && dvt <= 3.40282347e+38f;   // positive, normal, finite
    const float f = dnorm ? __builtin_amdgcn_frexp_mantf(dvt) : 0.5f;
    if constexpr (EDGE) {
      // sacc[kb][i] is key k0 + 4 h + 32 kb + 8 (i / 4) + i % 4. The allowed
      // keys of a query are one range [lo, hi] (below N; the causal or band
      // upper edge; the band lower edge), computed once per lane; each
      // element then needs two compares against a constant.
      const int base = k0 + 4 * h;
      const int w = min(window, N);   // a band wider than N cuts nothing
      int hi = N - 1;
      if (causal) hi = min(hi, qrow);
      else if (window >= 0) hi = min(hi, qrow + w);
      const int lo = window >= 0 ? qrow - w : 0;
      const int ohi = hi - base, olo = lo - base;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = kb * 32 + 8 * (i >> 2) + (i & 3);
          if (off > ohi || off < olo) sacc[kb][i] = -INFINITY;
        }
    }
    float sv[16 * NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sv[16 * kb + i] = sacc[kb][i];
    float mx = halves_max(tree_max<16 * NKB>(sv));
    const float mxs = mx == -INFINITY ? -INFINITY : mx * c;
    const float mnew = max2(m, ceilf(mxs));
    const float muse = mnew == -INFINITY ? 0.f : mnew;
    m_ref = m_ref == -INFINITY ? mnew : m_ref;
    float shift = mnew == -INFINITY ? 0.f : mnew - m_ref;   // integer >= 0
    if (__ballot(shift > kMaxShift) != 0) {
      // rare: rebase O and l (all tiles so far: PV of the previous tile is
      // ordered before this) by an exact power of two
      const float f = shift > kMaxShift ? __builtin_ldexpf(1.f, -(int)shift) : 1.f;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) oacc[db] *= f;
      l *= f;
      m_ref = shift > kMaxShift ? mnew : m_ref;
      shift = shift > kMaxShift ? 0.f : shift;
    }
    sa[PB] = dnorm ? min(kE8M0One + dexp, 254) : 0;   // 255 is E8M0 NaN
    sb[PB] = kE8M0One + (int)shift;
    lf[PB] = __builtin_ldexpf(__builtin_amdgcn_rcpf(f), (int)shift);
    // stored value p * f * 2^8 = 2^(c s - (muse - 8 - log2 f))
    const float bias = muse - kPScaleLog2 - __builtin_amdgcn_logf(f);
    float ps[16 * NKB];
#pragma unroll
    for (int e = 0; e < 16 * NKB; ++e) {
      ps[e] = fast_exp2(fmaf(sv[e], c, -bias));
      if constexpr (EDGE) ps[e] = sv[e] == -INFINITY ? 0.f : ps[e];
    }
#pragma unroll
    for (int w = 0; w < 8 * NH; ++w)
      pbuf[PB][w / 8][w % 8] = cvt4(ps[4 * w], ps[4 * w + 1], ps[4 * w + 2], ps[4 * w + 3]);
    m = mnew;
  }

  __device__ __forceinline__ void sync_tiles() {
    wait_vmem();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
  }

  template <bool EDGE, int PB, bool FIRST>
  __device__ __forceinline__ void iteration(int j) {
    sync_tiles();                           // K_j, V_{j-1} landed; iteration j-1 done
    issue_k<PB ^ 1>(j + 1);                 // unconditional: see the bf16 kernel
    issue_v<PB>(j);
    // The V reads of the previous tile's first half follow the K reads: the
    // scheduling groups of the bf16-score QK^T take the LDS reads that precede
    // them, and with E4M3 scores this order also measured +1.3% (d = 128 and
    // 64, same-box A/B, bit-identical).
    read_k_qk<PB>();
    if constexpr (!FIRST) read_v<PB ^ 1>(0);
    if constexpr (!FIRST) pv_rest<PB ^ 1>();
    softmax<EDGE, PB>(j);
    __builtin_amdgcn_iglp_opt(0);
  }

  template <bool EDGE>
  __device__ __forceinline__ void run(int j0, int j1) {
    int j = j0;
    if (j < j1 && ((j - kt0) & 1)) iteration<EDGE, 1, false>(j++);
    for (; j + 1 < j1; j += 2) {
      iteration<EDGE, 0, false>(j);
      iteration<EDGE, 1, false>(j + 1);
    }
    if (j < j1) iteration<EDGE, 0, false>(j);
  }
};

// Q and K: E4M3 codes (uint8), or bf16 (uint16) when QBF. DQ and DK are
// unused when QBF. Every instance runs two workgroups per CU (two waves per
// SIMD, 256 registers each): the bf16-score instance at d = 128, whose Q and K
// fragments are twice the size, fits since the softmax keeps no O rescale
// state (two spilled dwords, outside the tile loops).
template <int D, bool QBF>
__global__ __launch_bounds__(kThreads, 2)
void attn_fwd_fp8_kernel(const void* __restrict__ Qv, const void* __restrict__ Kv,
                         const uint8_t* __restrict__ V, uint16_t* __restrict__ O,
                         float* __restrict__ LSE, const float* __restrict__ DQ,
                         const float* __restrict__ DK, const float* __restrict__ DV, int N,
                         int nqt, float c0, int causal, int window, int qsign) {
  using S = Fp8Fwd<D, QBF>;
  __shared__ __attribute__((aligned(1024))) char k0s[S::KTILE];
  __shared__ __attribute__((aligned(1024))) char k1s[S::KTILE];
  __shared__ __attribute__((aligned(1024))) char v0s[S::VTILE];
  __shared__ __attribute__((aligned(1024))) char v1s[S::VTILE];

  S st;
  st.kl[0] = (lds_char*)k0s;
  st.kl[1] = (lds_char*)k1s;
  st.vl[0] = (lds_char*)v0s;
  st.vl[1] = (lds_char*)v1s;
  const TileRange tr = tile_range(N, nqt, causal, window, kBM, S::BN);
  st.N = N;
  st.causal = causal;
  st.window = window;
  st.kt0 = tr.kt0;
  st.kt1 = tr.kt1;
  const int tid = threadIdx.x;
  st.lane = tid & 63;
  st.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  st.h = st.lane >> 5;
  st.l32 = st.lane & 31;
  st.qrow = tr.q0 + st.wave * 32 + st.l32;
  st.krow = st.l32 * D;
  st.kswz = swz_k8<D>(st.l32) << 4;
  const size_t head = (size_t)tr.bh * N * D;
  const int nsb = (N + 127) / 128;             // scaling blocks per head
  st.dk = QBF ? nullptr : DK + (size_t)tr.bh * nsb;
  st.dv = DV + (size_t)tr.bh * nsb;
  st.cq = QBF ? c0 : c0 * DQ[(size_t)tr.bh * nsb + tr.q0 / 128];

  if constexpr (QBF) {
    // Q fragments (bf16): lane holds q[qrow][16t + 8h .. +7].
    const uint16_t* Q = (const uint16_t*)Qv;
#pragma unroll
    for (int t = 0; t < S::KSTEPS; ++t) {
      i32x4 x = {0, 0, 0, 0};
      if (st.qrow < N) x = *(const i32x4*)(Q + head + (size_t)st.qrow * D + 16 * t + 8 * st.h);
      x ^= qsign;
      st.qf[t] = __builtin_bit_cast(bf16x8, x);
    }
  } else {
    // Q fragments (E4M3): lane holds q8[qrow][64t + 32h .. +31].
    const uint8_t* Q = (const uint8_t*)Qv;
#pragma unroll
    for (int t = 0; t < S::KSTEPS; ++t) {
      i32x4 x0 = {0, 0, 0, 0}, x1 = {0, 0, 0, 0};
      if (st.qrow < N) {
        const uint8_t* p = Q + head + (size_t)st.qrow * D + 64 * t + 32 * st.h;
        x0 = *(const i32x4*)p;
        x1 = *(const i32x4*)(p + 16);
      }
      x0 ^= qsign;
      x1 ^= qsign;
      st.qf[t] = i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    }
  }

  // HBM -> LDS copies: LDS chunk p (p = 64 * block + lane) of the K image is
  // row p / KDCH, physical column p % KDCH, holding logical column
  // (p % KDCH) ^ swizzle(row). The V image's LDS row r holds key v8_row(r).
  st.kres = make_rsrc((const char*)Kv + head * S::KBYTES, (uint32_t)N * D * S::KBYTES);
  st.vres = make_rsrc(V + head, (uint32_t)N * D);
  {
    const int p = st.wave * 64 + st.lane;        // chunk of copy round 0
    const int row = p / S::KDCH, pc = p % S::KDCH;
    if constexpr (QBF) st.koff = row * D * 2 + (pc ^ bf16_swz_k<D>(row)) * 16;
    else st.koff = row * D + (pc ^ swz_k8<D>(row)) * 16;
    const int vrow = p / S::VDCH, vpc = p % S::VDCH;
    st.voff = v8_row(vrow) * D + (vpc ^ swz_v8<D>(vrow)) * 16;
  }

#pragma unroll
  for (int db = 0; db < S::DBLK; ++db) st.oacc[db] = f32x16{};
  st.l = 0.f;
  st.ones = ones_operand(st.lane);
  st.m = -INFINITY;
  st.m_ref = -INFINITY;
  st.sa[0] = st.sa[1] = kE8M0One;
  st.sb[0] = st.sb[1] = kE8M0One;
  st.lf[0] = st.lf[1] = 0.f;

  const int kt0 = tr.kt0, kt1 = tr.kt1;

  if (kt0 < kt1) {
    st.template issue_k<0>(kt0);
    const InteriorSpan span = interior_span(tr, N, causal, window, S::BN);
    if (kt0 < span.ia || kt0 >= span.ib) st.template iteration<true, 0, true>(kt0);
    else st.template iteration<false, 0, true>(kt0);
    const int a = min(max(span.ia, kt0 + 1), kt1), b = min(max(span.ib, a), kt1);
    st.template run<true>(kt0 + 1, a);
    st.template run<false>(a, b);
    st.template run<true>(b, kt1);
    st.sync_tiles();
    if ((kt1 - 1 - kt0) & 1) {
      st.template read_v<1>(0);
      st.template pv_rest<1>();
    } else {
      st.template read_v<0>(0);
      st.template pv_rest<0>();
    }
  }

  // ---- epilogue: O = O_acc / l and LSE = ln 2 * (m_ref + log2(l) - 8)
  const float lt = st.l;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (st.qrow < N) {
    uint16_t* orow = O + head + (size_t)st.qrow * D;
#pragma unroll
    for (int db = 0; db < S::DBLK; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(st.oacc[db][4 * g4 + e] * inv);
        *(bf16x4*)(orow + db * 32 + 8 * g4 + 4 * st.h) = o4;
      }
    if (st.h == 0)
      LSE[(size_t)tr.bh * N + st.qrow] =
          lt > 0.f ? (st.m_ref + log2f(lt) - kPScaleLog2) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_attn_fwd_fp8(const FwdArgs& a, bool qk_bf16, hipStream_t stream) {
  const int nqt = (a.N + kBM - 1) / kBM;
  const int G = nqt * a.BH;  // bounded by the C ABI's shape checks
  const float c0 = fabsf(a.scale) * kLog2e;
  const bool neg = a.scale < 0.f;
  const uint8_t* v = (const uint8_t*)a.v;
  uint16_t* o = (uint16_t*)a.o;
  if (qk_bf16) {
    const int qsign = neg ? (int)0x80008000u : 0;
    if (a.d == 128)
      hipLaunchKernelGGL((attn_fwd_fp8_kernel<128, true>), dim3(G), dim3(kThreads), 0, stream, a.q,
                         a.k, v, o, a.lse, a.dq, a.dk, a.dv, a.N, nqt, c0, a.causal, a.window, qsign);
    else
      hipLaunchKernelGGL((attn_fwd_fp8_kernel<64, true>), dim3(G), dim3(kThreads), 0, stream, a.q,
                         a.k, v, o, a.lse, a.dq, a.dk, a.dv, a.N, nqt, c0, a.causal, a.window, qsign);
  } else {
    const int qsign = neg ? (int)0x80808080u : 0;
    if (a.d == 128)
      hipLaunchKernelGGL((attn_fwd_fp8_kernel<128, false>), dim3(G), dim3(kThreads), 0, stream, a.q,
                         a.k, v, o, a.lse, a.dq, a.dk, a.dv, a.N, nqt, c0, a.causal, a.window, qsign);
    else
      hipLaunchKernelGGL((attn_fwd_fp8_kernel<64, false>), dim3(G), dim3(kThreads), 0, stream, a.q,
                         a.k, v, o, a.lse, a.dq, a.dk, a.dv, a.N, nqt, c0, a.causal, a.window, qsign);
  }
  return hipGetLastError();
}

}  // namespace mi355attn
