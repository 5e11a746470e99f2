// Fused attention forward, bf16 inputs, for gfx950 (MI355X / CDNA4).
//
// A workgroup of NW waves (4, or 8 for large unwindowed grids at d = 128)
// owns NW x 32 x QB queries of one (batch, head): each wave owns QB blocks of
// 32 queries. It streams the allowed key/value tiles (BN keys each) through
// LDS. Scores, probabilities and the output
// accumulator never leave registers; the N x N score matrix is never formed.
// This is the tiled, fused scheme of [WGC] sections 1-2 (QK^T -> softmax
// statistics -> PV with running max/sum and output rescale) and [YT] sections
// 1.2 and 2.1.1 (softmax + mask + matmul in one kernel; global tile ->
// shared-memory tile -> register tile), mapped onto CDNA4 rather than Hopper:
//
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16. In the transposed product each
//    lane holds 16 keys of ONE query, so a row's max and sum are in-lane
//    reductions plus one v_permlane32_swap with the lane holding the other 16.
//  * The probabilities leave the accumulator already in the B-operand layout
//    of O^T = V^T P^T: P never moves between lanes and never touches LDS (the
//    register hand-off between the two GEMMs of [WGC] section 1). The V^T
//    operand is read with ds_read_b64_tr_b16, gfx950's transposing LDS read.
//  * K and V tiles are copied HBM -> LDS by buffer_load_dwordx4 ... lds (no
//    staging registers, no LDS write instructions; rows past N read as zero
//    through the buffer's range check). Tile j+1's K and tile j's V are in
//    flight while tile j is multiplied (double buffers: [JJ] section 1.2's
//    ping-pong buffers, [WGC]'s prefetch of the next KV block). The barrier
//    between tiles carries no memory fence, so those copies stay in flight.
//  * Software pipeline inside the wave ([JJ] section 2.2, GEMM/softmax
//    overlap). Iteration j: the MFMAs of S(j) = K_j Q^T, with each K fragment
//    read from LDS a fixed number of k-steps ahead of its MFMA (scheduling
//    groups), then the V_{j-1} fragments and the MFMAs of O += P(j-1) V_{j-1}
//    interleaved with the softmax of S(j), so the exponentials run while the
//    matrix cores are busy (interleaving independent VALU work into a wave's
//    own MFMA stream is what the SIMD overlaps; a VALU-only wave beside an
//    MFMA-only wave is not). P alternates between two register sets.
//  * Online softmax in base 2 with log2(e) folded into the scale (v_exp_f32
//    computes 2^x). A tile is first exponentiated against the row's current
//    reference max; only if some lane's sum of p exceeds a bound (first tile,
//    scores far above the reference, Inf/NaN) does the wave compute the row
//    max, move the reference (when the max exceeds it by more than 8) and
//    redo the tile. So the row max and the O rescale (owed to the next
//    iteration, before its PV) are rare; O / l and the LSE are unchanged.
//  * Key tiles wholly outside the causal / sliding-window band are never
//    visited ([YT] section 2.1.2); only tiles straddling the band's edge or the
//    ragged end of the sequence carry mask code.
//  * Workgroup ids are remapped so the query tiles of one head land on one XCD
//    and share K/V in its L2. Causal problems issue their heaviest tiles
//    first; banded ones go in ascending order, so a tile's first key tiles
//    are still in L2 from the tile before. Short causal problems give each
//    workgroup the tiles p and nqt-1-p of a head, so every workgroup carries
//    the same work; the second tile's Q loads and first K copy overlap the
//    first tile's drain.
// The kernel state lives in one struct whose members are all force-inlined, so
// every array is promoted to registers.
#include "attn_device.h"
#include "attn_internal.h"

namespace mi355attn {
namespace {

constexpr float kRescaleSlack = 8.f;   // see the header comment

template <int D, int BN, int QB, int NW>
struct Bf16Fwd {
  static constexpr int THREADS = 64 * NW;               // NW waves per workgroup
  static constexpr int DCH = D / 8;                     // 16-byte chunks per row
  static constexpr int KSTEPS = D / 16;                 // MFMA k-steps of QK^T
  static constexpr int DBLK = D / 32;                   // 32-wide d blocks of O^T
  static constexpr int NKB = BN / 32;                   // 32-key blocks of S^T
  static constexpr int PST = BN / 16;                   // 16-key MFMA steps of PV
  static constexpr int TILE = BN * D * 2;               // bytes of one K or V tile
  static constexpr int LOADS = TILE / (16 * THREADS);   // 16-byte copies per thread
  static_assert(LOADS * 16 * THREADS == TILE, "tile must split into whole copies per thread");
  // Largest accepted sum of one lane's p without a new reference max: with
  // the exact step's slack every p <= 2^8, so this is never exceeded
  // right after it; it bounds every p by 16 NKB 2^8.
  static constexpr float kFastLimit = 16.f * NKB * 256.f;

  // problem
  lds_char* kl[2];   // K stages: K_t lives in stage (t - kt0) & 1
  lds_char* vl[2];   // V stages, same rule
  int N, causal, window, kt0, kt1;
  float c;
  int lane, wave, h, l32;
  int qrow[QB];
  i32x4 kres, vres;                  // buffer descriptors of this head's K and V
  int koff[LOADS], voff[LOADS];
  // state
  bf16x8 qf[QB][KSTEPS];
  f32x16 oacc[QB][DBLK];
  f32x16 sacc[QB][NKB];
  bf16x8 pbuf[2][QB][PST];
  // V fragments of the 64-key tile at d = 128 are streamed from LDS one
  // 16-key step at a time, right before their MFMAs (a whole tile's would not
  // fit two waves per SIMD); other tiles read theirs together. K fragments are
  // read inside the scheduled QK^T (qk).
  static constexpr bool STREAM = D == 128 && BN == 64;
  static constexpr bool kRescaleFirst = D == 256;
  bf16x8 vf[STREAM ? 1 : PST][DBLK];
  float m[QB], l[QB], alpha[QB];
  bool owe_rescale;

  template <int ST>
  __device__ __forceinline__ void issue_k(int kt) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u)
      copy_to_lds16(kres, kl[ST] + (u * NW + wave) * 1024, koff[u], (int)((uint32_t)kt * (BN * D * 2)));
  }
  template <int ST>
  __device__ __forceinline__ void issue_v(int kt) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u)
      copy_to_lds16(vres, vl[ST] + (u * NW + wave) * 1024, voff[u], (int)((uint32_t)kt * (BN * D * 2)));
  }

  // A operand of S^T = K Q^T for 32-key block kb, k-step t: lane holds
  // K[32 kb + l32][16 t + 8 h .. +7].
  template <int ST>
  __device__ __forceinline__ bf16x8 k_frag(int kb, int t) const {
    const int row = kb * 32 + l32;
    const int ch = 2 * t + h;
    return *(const lds_bf16x8*)(kl[ST] + row * D * 2 + ((ch ^ bf16_swz_k<D>(row)) << 4));
  }
  // A operand of O^T += V^T P^T for MFMA step s (into fragment set i): lane
  // (d, h) holds V at keys 16 s + 4 h + 0..3 and + 8 (the key order of the
  // S^T accumulator).
  template <int ST>
  __device__ __forceinline__ void read_v_step(int s, int i) {
    const lds_char* Vs = vl[ST];
    const int g = lane >> 4, sl = lane & 15;
    const int r1 = 16 * s + 4 * (g >> 1) + (sl >> 2);
    const int r2 = r1 + 8;
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const int col = db * 32 + 16 * (g & 1) + 4 * (sl & 3);
      const int a1 = r1 * D * 2 + (((col >> 3) ^ bf16_swz_v<D>(r1)) << 4) + ((col >> 2) & 1) * 8;
      const int a2 = r2 * D * 2 + (((col >> 3) ^ bf16_swz_v<D>(r2)) << 4) + ((col >> 2) & 1) * 8;
      const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Vs + a1));
      const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Vs + a2));
      vf[i][db] = __builtin_bit_cast(bf16x8, i16x8{v1[0], v1[1], v1[2], v1[3], v2[0], v2[1],
                                                   v2[2], v2[3]});
    }
  }
  template <int ST>
  __device__ __forceinline__ void read_v() {
    if constexpr (!STREAM) {
#pragma unroll
      for (int s = 0; s < PST; ++s) read_v_step<ST>(s, s);
    }
  }

  // K fragments in flight ahead of the MFMAs that use them, in k-steps of
  // NKB QB MFMAs each (same-box sweeps of 2 .. 6 with QB = 1: d = 128 with
  // 64-key tiles 3, with 32-key tiles 6; d = 64: 2; d = 256: 4).
  static constexpr int kKAhead = NKB == 2 ? (D == 64 ? 2 : 3) : (D == 256 ? 4 : 6);

  // S^T of the tile in K stage ST.
  template <int ST>
  __device__ __forceinline__ void qk() {
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sacc[b][kb] = f32x16{};
    // The 32-key blocks' accumulator chains advance together, k-step by
    // k-step, and each step's K fragments are read kKAhead steps before their
    // MFMAs. Left to itself the compiler streams a block's fragments through
    // one register set, or waits for all reads before the first MFMA, so
    // MFMAs wait whole LDS round trips. Same-box A/B, bit-identical outputs:
    // +2.0 .. 2.8% at B16 H16 N8192, +4.4% causal B4 H16 N2048, +2.5% causal
    // B16 H16 N8192, +3.9 .. 4.2% causal window 1024 at d = 64, +2.7 .. 3% at
    // d = 256.
    bf16x8 f[KSTEPS][NKB];
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) f[t][kb] = k_frag<ST>(kb, t);
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int b = 0; b < QB; ++b)
          sacc[b][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[t][kb], qf[b][t], sacc[b][kb], 0, 0, 0);
    // scheduling groups (0x100 = LDS reads, 0x008 = MFMAs) take the
    // instructions that precede them, so the V reads of an iteration come
    // after this function
    __builtin_amdgcn_sched_group_barrier(0x100, NKB * kKAhead, 0);
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, NKB * QB, 0);
      if (t + kKAhead < KSTEPS) __builtin_amdgcn_sched_group_barrier(0x100, NKB, 0);
    }
  }

  // O^T += V^T P^T with P set PB and the V tile in stage PB.
  template <int PB>
  __device__ __forceinline__ void pv() {
#pragma unroll
    for (int s = 0; s < PST; ++s) {
      if constexpr (STREAM) read_v_step<PB>(s, 0);
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int b = 0; b < QB; ++b)
          oacc[b][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[STREAM ? 0 : s][db], pbuf[PB][b][s],
                                                                oacc[b][db], 0, 0, 0);
    }
  }

  // Disallowed keys of an edge tile get score -inf. sacc[b][kb][i] is the
  // score of key base + 32 kb + 8 (i/4) + i%4 (base = k0 + 4 h) against query
  // qrow[b]. The allowed keys of a query form one range [lo, hi] (below N;
  // the causal or band upper edge; the band lower edge), so each lane
  // computes that range once per tile and each element needs two compares
  // against a constant offset.
  __device__ __forceinline__ void mask(int kt) {
    const int base = kt * BN + 4 * h;
    const int w = min(window, N);   // a band wider than N cuts nothing
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      int hi = N - 1;
      if (causal) hi = min(hi, qrow[b]);
      else if (window >= 0) hi = min(hi, qrow[b] + w);
      const int lo = window >= 0 ? qrow[b] - w : 0;
      const int ohi = hi - base, olo = lo - base;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = kb * 32 + 8 * (i >> 2) + (i & 3);
          if (off > ohi || off < olo) sacc[b][kb][i] = -INFINITY;
        }
    }
  }

  // P set PB of query block b = bf16(2^(c s - muse)); returns this lane's sum
  // of the rounded values (the ones PV multiplies). c > 0 always (a zero
  // scale zeroes Q instead), so a masked key's -inf score gives p = 0.
  template <int PB>
  __device__ __forceinline__ float exponentiate(int b, float muse) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(sacc[b][kb][i], c, -muse));
        pbuf[PB][b][kb * 2 + (i >> 3)][i & 7] = (__bf16)p;
      }
    float part[PST];
#pragma unroll
    for (int st = 0; st < PST; ++st) part[st] = sum_bf16x8(pbuf[PB][b][st], 0.f);
    float rs = part[0];
#pragma unroll
    for (int st = 1; st < PST; ++st) rs += part[st];
    return rs;
  }

  // Online softmax of S(kt) into P set PB.
  //
  // Common case: exponentiate against the current reference max m and accept
  // the tile if every lane's sum of its p stays <= kFastLimit (so each p is
  // bounded, and O, l need no rescale). No row max is computed.
  // Otherwise (first tile, a score far above m, Inf or NaN), the whole wave
  // takes the exact step: row max over both half-rows, m moves to it when it
  // exceeds m by more than kRescaleSlack, O's rescale is owed, P recomputed.
  template <bool EDGE, int PB, bool FIRST>
  __device__ __forceinline__ void softmax(int kt) {
    if constexpr (EDGE) mask(kt);
    if constexpr (!FIRST) {
      float rs[QB];
      bool over = false;
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        rs[b] = exponentiate<PB>(b, m[b]);
        over = over || !(rs[b] <= kFastLimit);
        // A row that has seen no allowed key yet (m = -inf) gives -inf + inf
        // for its masked keys here; it takes the exact step instead.
        if constexpr (EDGE) over = over || m[b] == -INFINITY;
      }
      if (__ballot(over) == 0) {
#pragma unroll
        for (int b = 0; b < QB; ++b) l[b] += rs[b];
        owe_rescale = false;
        return;
      }
    }
    bool grow_any = false;
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      float sv[16 * NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sv[16 * kb + i] = sacc[b][kb][i];
      const float mx = halves_max(tree_max<16 * NKB>(sv));
      const float mxs = mx == -INFINITY ? -INFINITY : mx * c;
      const bool grow = mxs > m[b] + kRescaleSlack;
      const float mnew = grow ? mxs : m[b];
      const float muse = mnew == -INFINITY ? 0.f : mnew;
      const float a = fast_exp2(m[b] - muse);
      const float rs = exponentiate<PB>(b, muse);
      l[b] = l[b] * a + rs;
      alpha[b] = a;
      m[b] = mnew;
      grow_any = grow_any || grow;
    }
    owe_rescale = __ballot(grow_any) != 0;
  }

  // O *= alpha, owed by the last softmax (rare).
  __device__ __forceinline__ void rescale() {
    if (owe_rescale) {
#pragma unroll
      for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int db = 0; db < DBLK; ++db) oacc[b][db] *= alpha[b];
    }
  }

  // Each wave waits for its own copies (vmcnt), then a barrier without a
  // memory fence: a fenced barrier would also wait for the copies of the next
  // tiles, which are meant to stay in flight. Separate LDS objects per stage
  // let the compiler see that this iteration's LDS reads and the copies in
  // flight never touch the same memory.
  __device__ __forceinline__ void sync_tiles() {
    wait_vmem();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
  }

  // Iteration j (stage PB = (j - kt0) & 1): copies of K_{j+1} and V_j go in
  // flight; S(j) = K_j Q^T; owed rescale; then PV(j-1) interleaved with the
  // softmax of S(j) into P set PB.
  template <bool EDGE, int PB, bool FIRST>
  __device__ __forceinline__ void iteration(int j) {
    sync_tiles();                           // K_j, V_{j-1} landed; iteration j-1 done
    // Unconditional (a branch here would make the compiler wait for every
    // copy at the join): past the last tile it fetches an unused tile, and
    // rows past N read as zero through the buffer range check.
    issue_k<PB ^ 1>(j + 1);
    issue_v<PB>(j);
    // At d = 256 (one workgroup per CU, registers to spare) the owed rescale
    // goes first, so QK^T, the V reads and PV share one scheduling region and
    // the V reads start under the QK^T MFMAs (+1.8% in a same-box A/B,
    // bit-identical). Elsewhere the V fragments this keeps live cost more
    // than the earlier reads gain (-2% at B16 H16 N8192 d128).
    if constexpr (kRescaleFirst) rescale();
    qk<PB>();
    if constexpr (!FIRST) read_v<PB ^ 1>();
    if constexpr (!kRescaleFirst) rescale();
    if constexpr (!FIRST) pv<PB ^ 1>();
    softmax<EDGE, PB, FIRST>(j);
    __builtin_amdgcn_iglp_opt(0);
  }

  // Tiles [j0, j1) with P set (j - kt0) & 1, unrolled by two so each P set
  // keeps its registers.
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

// PAIRED: each workgroup runs a causal tile pair (see TilePair); otherwise
// one query tile per workgroup (order: see tile_range).
// Workgroups per CU: two waves per SIMD (8 / NW workgroups), except the d = 64
// single-tile instance, which fits 168 registers with its tile loops free of
// spills and runs three 4-wave workgroups per CU: at d = 64 a workgroup has
// half the MFMA work per key tile, so its fixed entry and drain costs weigh
// more, and a third resident workgroup covers them (banded masks most).
template <int D, int BN, int QB, int NW, bool PAIRED>
constexpr int bf16_wg_per_cu() {
  if (QB != 1 || D > 128) return 1;
  return (D == 64 && NW == 4 && !PAIRED) ? 3 : 8 / NW;
}

template <int D, int BN, int QB, int NW, bool PAIRED>
__global__ __launch_bounds__(64 * NW, (bf16_wg_per_cu<D, BN, QB, NW, PAIRED>()))
void attn_fwd_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                          const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                          float* __restrict__ LSE, int N, int nqt, float c, int causal,
                          int window, int qsign, int qkeep) {
  using S = Bf16Fwd<D, BN, QB, NW>;
  constexpr int BMQ = NW * 32 * QB;
  __shared__ __attribute__((aligned(1024))) char k0s[S::TILE];
  __shared__ __attribute__((aligned(1024))) char k1s[S::TILE];
  __shared__ __attribute__((aligned(1024))) char v0s[S::TILE];
  __shared__ __attribute__((aligned(1024))) char v1s[S::TILE];

  S st;
  st.kl[0] = (lds_char*)k0s;
  st.kl[1] = (lds_char*)k1s;
  st.vl[0] = (lds_char*)v0s;
  st.vl[1] = (lds_char*)v1s;
  st.N = N;
  st.causal = causal;
  st.window = window;
  st.c = c;
  const int tid = threadIdx.x;
  st.lane = tid & 63;
  st.wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  st.h = st.lane >> 5;
  st.l32 = st.lane & 31;

  // HBM -> LDS copies. Chunk p of a tile's LDS image (16 B, p = 64 * block +
  // lane) sits at row p / DCH, physical column p % DCH, which holds logical
  // column (p % DCH) ^ swizzle(row); each lane fetches exactly that chunk.
#pragma unroll
  for (int u = 0; u < S::LOADS; ++u) {
    const int p = (u * NW + st.wave) * 64 + st.lane;
    const int row = p / S::DCH, pc = p % S::DCH;
    st.koff[u] = (row * D + (pc ^ bf16_swz_k<D>(row)) * 8) * 2;
    st.voff[u] = (row * D + (pc ^ bf16_swz_v<D>(row)) * 8) * 2;
  }

  // Base pointers are parked (see park) while the tiles run.
  const ParkedPtr<PAIRED> pq(Q), pk(K), pv(V), po(O), plse(LSE);

  // Query tile set-up: key-tile range, query rows, this head's K/V buffer
  // descriptors, the Q fragments (B operand of S^T = K Q^T: lane holds
  // q[qrow][16t + 8h .. +7]) and the copy of the first K tile into stage 0.
  // Called for a pair's second tile while the first one drains, so the Q
  // loads and the first copy are in flight during its last PV and epilogue.
  auto begin = [&](const TileRange& tr) __attribute__((always_inline)) {
    st.kt0 = tr.kt0;
    st.kt1 = tr.kt1;
#pragma unroll
    for (int b = 0; b < QB; ++b) st.qrow[b] = tr.q0 + st.wave * 32 * QB + 32 * b + st.l32;
    const size_t head = (size_t)tr.bh * N * D;
    const uint16_t* Qp = pq.template get<const uint16_t>();
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
      for (int t = 0; t < S::KSTEPS; ++t) {
        i32x4 x = {0, 0, 0, 0};
        if (st.qrow[b] < N) x = *(const i32x4*)(Qp + head + (size_t)st.qrow[b] * D + 16 * t + 8 * st.h);
        x = (x & qkeep) ^ qsign;  // zero Q for a zero scale; exact sign flip for a negative one
        st.qf[b][t] = __builtin_bit_cast(bf16x8, x);
      }
    st.kres = make_rsrc(pk.template get<const uint16_t>() + head, (uint32_t)N * D * 2);
    st.vres = make_rsrc(pv.template get<const uint16_t>() + head, (uint32_t)N * D * 2);
    if (tr.kt0 < tr.kt1) st.template issue_k<0>(tr.kt0);
  };

  TileRange tr;
  TilePair pair = {0, 0, -1};
  if constexpr (PAIRED) {
    pair = tile_pair(nqt);
    tr = tile_range_at(pair.bh, pair.first, N, causal, window, BMQ, BN);
  } else {
    tr = tile_range(N, nqt, causal, window, BMQ, BN);
  }
  begin(tr);

  for (;;) {
#pragma unroll
    for (int b = 0; b < QB; ++b) {
#pragma unroll
      for (int db = 0; db < S::DBLK; ++db) st.oacc[b][db] = f32x16{};
      st.m[b] = -INFINITY;   // reference max of c * s (base-2 units)
      st.l[b] = 0.f;         // running sum over this lane's keys
      st.alpha[b] = 1.f;
    }
    st.owe_rescale = false;

    const int kt0 = tr.kt0, kt1 = tr.kt1;
    const InteriorSpan span = interior_span(tr, N, causal, window, BN);
    int cur_bh = tr.bh, cur_q0 = tr.q0;   // for the epilogue
    if constexpr (PAIRED) {
      cur_bh = park(cur_bh);
      cur_q0 = park(cur_q0);
    }
    // A pair's second tile, if any, is set up while the first one drains.
    auto advance = [&]() __attribute__((always_inline)) {
      if constexpr (PAIRED) {
        if (pair.second >= 0) {
          tr = tile_range_at(pair.bh, pair.second, N, causal, window, BMQ, BN);
          pair.second = -1;
          begin(tr);
          return true;
        }
      }
      return false;
    };
    bool more;
    if (kt0 < kt1) {
      // the first tile has no PV yet
      if (kt0 < span.ia || kt0 >= span.ib) st.template iteration<true, 0, true>(kt0);
      else st.template iteration<false, 0, true>(kt0);
      const int a = min(max(span.ia, kt0 + 1), kt1), b = min(max(span.ib, a), kt1);
      st.template run<true>(kt0 + 1, a);
      st.template run<false>(a, b);
      st.template run<true>(b, kt1);
      // drain: PV of the last tile. After this barrier no wave reads either K
      // stage again, so the next query tile's first K copy may start.
      st.sync_tiles();
      more = advance();
      st.rescale();
      if ((kt1 - 1 - kt0) & 1) {
        st.template read_v<1>();
        st.template pv<1>();
      } else {
        st.template read_v<0>();
        st.template pv<0>();
      }
    } else {
      more = advance();
    }

    // ---- epilogue: O = O^T / l (bf16, RNE), LSE = ln 2 * (m + log2 l)
    const size_t head = (size_t)cur_bh * N * D;
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const int qrow = cur_q0 + st.wave * 32 * QB + 32 * b + st.l32;
      const float lt = halves_sum(st.l[b]);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      if (qrow < N) {
        uint16_t* orow = po.template lanes<uint16_t>() + head + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < S::DBLK; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            bf16x4 o4;
#pragma unroll
            for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(st.oacc[b][db][4 * g4 + e] * inv);
            *(bf16x4*)(orow + db * 32 + 8 * g4 + 4 * st.h) = o4;
          }
        if (st.h == 0) {
          const float muse = st.m[b] == -INFINITY ? 0.f : st.m[b];
          plse.template lanes<float>()[(size_t)cur_bh * N + qrow] = lt > 0.f ? (muse + log2f(lt)) * kLn2 : -INFINITY;
        }
      }
    }
    if (!more) break;
  }
}

// Configuration per head dimension: queries per wave (32 QB), keys per tile.
// At d = 128 the 8-wave workgroups take 64-key tiles (fragments streamed,
// see Bf16Fwd::STREAM): half the barriers and half the per-tile softmax
// bookkeeping per key (+2.0 .. 2.4% at B16 H16 N8192 in a same-box A/B).
// The 4-wave ones keep 32: there 64 measured -1% causal at N 8192.
constexpr int kQB128 = 1, kBN128 = 32, kBN128Wide = 64;
constexpr int kQB64 = 1, kBN64 = 64;
// d = 256: 128 accumulator floats per lane and 64-register Q, K and V
// fragment sets need more than the 256 registers of two waves per SIMD; one
// workgroup per CU gets the whole register file.
constexpr int kQB256 = 1, kBN256 = 32;

// Waves per workgroup at d = 128 (two waves per SIMD either way): one 8-wave
// workgroup per CU copies each K/V tile into LDS once for 256 queries, half
// the L2 -> LDS traffic and LDS writes of two 4-wave workgroups. Used for
// unmasked problems only (with a causal or window mask, the uneven work per
// query tile balances worse over half as many, twice as large tiles) and when
// there are at least this many 256-query tiles, so that the grid still fills
// the CUs.
constexpr long long kWideGridMin = 1024;

// Causal problems of at most this many 128-query tiles per head run tile
// pairs. Pairs halve the number of workgroups and give them equal work, which
// pays where the tiles are short (nqt+1 key-tile rows per pair). With more
// tiles, the second tiles of the pairs start out of step and lose the shared
// K/V stream in L2, while the heaviest-first order already balances the
// grid. Windowed tiles carry near-equal work, so pairing buys nothing there.
constexpr int kPairMaxTiles = 32;

// One workgroup per tile pair (PAIRED) or per query tile.
template <int D, int BN, int QB, int NW, bool PAIRED>
void launch_cfg(const FwdArgs& a, float c, int qsign, int qkeep, hipStream_t stream) {
  const int rows = 32 * NW * QB;
  const int nqt = (a.N + rows - 1) / rows;
  const int per_head = PAIRED ? (nqt + 1) / 2 : nqt;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, BN, QB, NW, PAIRED>), dim3(per_head * a.BH),
                     dim3(64 * NW), 0, stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                     (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, a.N, nqt, c, a.causal, a.window,
                     qsign, qkeep);
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  // c = |scale| log2(e) > 0. A zero scale zeroes Q instead (every score 0,
  // exactly), so that a masked score of -inf times c stays -inf.
  const float c = a.scale == 0.f ? 1.f : fabsf(a.scale) * kLog2e;
  const int qsign = a.scale < 0.f ? (int)0x80008000u : 0;
  const int qkeep = a.scale == 0.f ? 0 : -1;
  const bool wide = !a.causal && a.window < 0 &&
                    (long long)((a.N + 255) / 256) * a.BH >= kWideGridMin;
  const bool pair = a.causal && a.window < 0 && (a.N + 127) / 128 <= kPairMaxTiles;
  if (a.d == 128) {
    if (wide) launch_cfg<128, kBN128Wide, kQB128, 8, false>(a, c, qsign, qkeep, stream);
    else if (pair) launch_cfg<128, kBN128, kQB128, 4, true>(a, c, qsign, qkeep, stream);
    else launch_cfg<128, kBN128, kQB128, 4, false>(a, c, qsign, qkeep, stream);
  } else if (a.d == 256) {
    launch_cfg<256, kBN256, kQB256, 4, false>(a, c, qsign, qkeep, stream);
  } else {
    if (pair) launch_cfg<64, kBN64, kQB64, 4, true>(a, c, qsign, qkeep, stream);
    else launch_cfg<64, kBN64, kQB64, 4, false>(a, c, qsign, qkeep, stream);
  }
  return hipGetLastError();
}

}  // namespace mi355attn
