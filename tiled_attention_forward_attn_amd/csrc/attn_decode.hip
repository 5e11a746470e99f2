// Attention of a few queries (Nq <= 32) against a long key/value sequence,
// for gfx950: decoding with a key/value cache ([JJ] section 3). The queries
// are the sequence's last Nq positions (query i at Nk - Nq + i; with causal
// masking it sees keys j <= Nk - Nq + i).
//
// Split-KV: the keys of every (batch, head) are cut into S contiguous chunks.
// One wave owns one (batch, head, chunk) and computes, over that chunk alone,
// the tiled online softmax of the prefill kernels ([WGC] sections 1-2): S^T =
// K Q^T on v_mfma_f32_32x32x16_bf16 (the queries fill one 32-wide MFMA block,
// rows past Nq are zero), the exact running max per tile, P in bf16 straight
// from the accumulator as the B operand of O^T += V^T P^T (V^T read with
// ds_read_b64_tr_b16). It writes the chunk's normalised output and its
// log-sum-exp as an fp32 partial; attn_lse_merge's kernel then combines the
// S partials of every row.
//
// The work is a stream of K and V through HBM: every wave copies its own
// tiles HBM -> LDS (global_load_lds_dwordx4 ... nt for tiles wholly inside
// the sequence, buffer_load_dwordx4 ... lds with its range check for the
// others) into a private double buffer (tile t+1 in flight while tile t is
// multiplied), so waves never wait for each other and the kernel has no
// barrier. One wave per workgroup
// lets up to five waves with their copies in flight share a CU.
//
// Paged cache (the PagedAttention cache management that [WGC] lists among its
// follow-up directions): the keys and values of a sequence sit in fixed-size
// pages of a shared pool [num_pages][H][page_size][d], and the sequence's
// block table names the page holding each run of page_size positions. The
// page size is a power of two no smaller than the 32-key tile, so a tile lies
// in one page: per tile one scalar table read, then a buffer descriptor over
// exactly that tile's rows, so the same copies and LDS layout serve both
// caches. Rows past the sequence (stale page contents) and table entries
// outside the pool read as zero through the descriptor's range check; no
// table content can make the kernel read outside the pool.
#include "attn_device.h"
#include "attn_internal.h"

namespace mi355attn {
namespace {

template <int D, int BN, bool PAGED>
struct DecodeWave {
  static constexpr int DCH = D / 8;          // 16-byte chunks per row
  static constexpr int KSTEPS = D / 16;
  static constexpr int DBLK = D / 32;
  static constexpr int NKB = BN / 32;
  static constexpr int PST = BN / 16;
  static constexpr int TILE = BN * D * 2;    // bytes of one K or V tile
  static constexpr int LOADS = TILE / 1024;  // 16-byte copies per lane per tile
  static_assert(LOADS * 1024 == TILE, "tile must split into 1 KiB wave copies");

  lds_char* kl[2];
  lds_char* vl[2];
  int Nq, Nk, causal, k_hi, lane, h, l32, qrow;
  float c;
  i32x4 kres, vres;
  int koff[LOADS], voff[LOADS];
  // paged cache: pool base, this sequence's block table row (read through the
  // constant address space, so a scalar load that the copies' vmcnt waits do
  // not drain) and this head; page_next is the page of the next tile to issue,
  // read one tile ahead
  const uint16_t* kpool;
  const uint16_t* vpool;
  const uint16_t* kg;   // contiguous cache: this head's K and V
  const uint16_t* vg;
  const __attribute__((address_space(4))) int* table;
  int head, H, page_shift, num_pages, page_next;

  __device__ __forceinline__ int load_page(int t) const {
    const int p0 = t * BN;
    return p0 < k_hi ? table[p0 >> page_shift] : -1;
  }
  bf16x8 qf[KSTEPS];
  f32x16 oacc[DBLK];
  f32x16 sacc[NKB];
  bf16x8 pbuf[PST];
  float m, l;

  // Tile t's copies. A tile whose BN rows all lie below k_hi (and, paged, on
  // a page inside the pool) is read with nontemporal flat loads: its rows are
  // inside the allocation by construction. Every other tile (the chunk's
  // ragged end, the unused tile past it, pages outside the pool) goes through
  // buffer descriptors, whose range check reads zeros.
  template <int ST>
  __device__ __forceinline__ void issue(int t) {
    const int p0 = t * BN;
    if constexpr (PAGED) {
      const int page = page_next;
      if (p0 + BN <= k_hi && (unsigned)page < (unsigned)num_pages) {
        page_next = load_page(t + 1);
        const size_t row = ((size_t)page * H + head) * ((size_t)1 << page_shift) +
                           (p0 & ((1 << page_shift) - 1));
        const char* kb = (const char*)(kpool + row * D);
        const char* vb = (const char*)(vpool + row * D);
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {
          copy_to_lds16_nt(kb + koff[u], kl[ST] + u * 1024);
          copy_to_lds16_nt(vb + voff[u], vl[ST] + u * 1024);
        }
        return;
      }
    } else {
      if (p0 + BN <= k_hi) {
        const char* kb = (const char*)kg + (size_t)t * TILE;
        const char* vb = (const char*)vg + (size_t)t * TILE;
#pragma unroll
        for (int u = 0; u < LOADS; ++u) {
          copy_to_lds16_nt(kb + koff[u], kl[ST] + u * 1024);
          copy_to_lds16_nt(vb + voff[u], vl[ST] + u * 1024);
        }
        return;
      }
    }
    int soff = (int)((uint32_t)t * TILE);
    if constexpr (PAGED) {
      // descriptors over tile t's rows of its page; zero rows past k_hi
      uint32_t bytes = 0;
      const uint16_t* kb = kpool;
      const uint16_t* vb = vpool;
      const int page = page_next;   // tile t's page (-1 past the chunk)
      page_next = load_page(t + 1);
      if (p0 < k_hi) {
        if ((unsigned)page < (unsigned)num_pages) {
          const size_t row = ((size_t)page * H + head) * ((size_t)1 << page_shift) +
                             (p0 & ((1 << page_shift) - 1));
          kb = kpool + row * D;
          vb = vpool + row * D;
          bytes = (uint32_t)min(BN, k_hi - p0) * D * 2;
        }
      }
      kres = make_rsrc(kb, bytes);
      vres = make_rsrc(vb, bytes);
      soff = 0;
    }
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      copy_to_lds16(kres, kl[ST] + u * 1024, koff[u], soff);
      copy_to_lds16(vres, vl[ST] + u * 1024, voff[u], soff);
    }
  }

  template <int ST>
  __device__ __forceinline__ void qk() {
    const lds_char* Ks = kl[ST];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int row = kb * 32 + l32;
      sacc[kb] = f32x16{};
#pragma unroll
      for (int t = 0; t < KSTEPS; ++t) {
        const int ch = 2 * t + h;
        const bf16x8 kf = *(const lds_bf16x8*)(Ks + row * D * 2 + ((ch ^ bf16_swz_k<D>(row)) << 4));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], sacc[kb], 0, 0, 0);
      }
    }
  }

  template <int ST>
  __device__ __forceinline__ void pv() {
    const lds_char* Vs = vl[ST];
    const int g = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int s = 0; s < PST; ++s) {
      const int r1 = 16 * s + 4 * (g >> 1) + (sl >> 2);
      const int r2 = r1 + 8;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const int col = db * 32 + 16 * (g & 1) + 4 * (sl & 3);
        const int a1 = r1 * D * 2 + (((col >> 3) ^ bf16_swz_v<D>(r1)) << 4) + ((col >> 2) & 1) * 8;
        const int a2 = r2 * D * 2 + (((col >> 3) ^ bf16_swz_v<D>(r2)) << 4) + ((col >> 2) & 1) * 8;
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Vs + a1));
        const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Vs + a2));
        const bf16x8 vf = __builtin_bit_cast(
            bf16x8, i16x8{v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]});
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pbuf[s], oacc[db], 0, 0, 0);
      }
    }
  }

  // Online softmax of one tile (exact running max; this kernel is bound by
  // HBM, not by the vector work): masked keys are those past the chunk's end
  // and, with causal masking, past the query's position.
  __device__ __forceinline__ void softmax(int t) {
    const int k0 = t * BN;
    const int klim = causal ? min(k_hi, Nk - Nq + qrow + 1) : k_hi;   // keys < klim allowed
    float sv[16 * NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
        sv[16 * kb + i] = key < klim ? sacc[kb][i] : -INFINITY;
      }
    const float mx = halves_max(tree_max<16 * NKB>(sv));
    const float mxs = mx == -INFINITY ? -INFINITY : mx * c;
    const float mnew = max2(m, mxs);
    const float muse = mnew == -INFINITY ? 0.f : mnew;
    const float a = fast_exp2(m - muse);
#pragma unroll
    for (int e = 0; e < 16 * NKB; ++e) {
      const float p = sv[e] == -INFINITY ? 0.f : fast_exp2(fmaf(sv[e], c, -muse));
      pbuf[e >> 3][e & 7] = (__bf16)p;
    }
    float rs = 0.f;
#pragma unroll
    for (int st = 0; st < PST; ++st) rs = sum_bf16x8(pbuf[st], rs);
    l = l * a + rs;
    m = mnew;
    if (__ballot(a != 1.f)) {
#pragma unroll
      for (int db = 0; db < DBLK; ++db) oacc[db] *= a;
    }
  }

  template <int P>
  __device__ __forceinline__ void tile(int t) {
    // stage P^1 held tile t-1, whose LDS reads the MFMAs below consumed
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    issue<P ^ 1>(t + 1);            // past the chunk it fetches unused keys (zeros past Nk)
    wait_vmem_upto<2 * LOADS>();     // tile t landed
    qk<P>();
    softmax(t);
    pv<P>();
  }
};

// Paged cache description (kernel argument).
struct PagedCache {
  const int* block_table;   // [B][max_pages]
  const int* seq_lens;      // [B]
  int H, num_pages, page_shift, max_pages;
};

// One wave per workgroup; workgroup w owns (bh, chunk) = (w / S, w % S).
// Contiguous cache: K, V [BH][Nk][d] and a fixed chunk. Paged: K, V are the
// pools, Nk and the chunk come from the sequence's length.
template <int D, int BN, bool PAGED>
__global__ __launch_bounds__(64)
void attn_decode_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                        const uint16_t* __restrict__ V, float* __restrict__ OP,
                        float* __restrict__ LP, int Nq, int Nk, int S, int chunk, float c,
                        int causal, int qsign, long long rows, PagedCache pc) {
  using W = DecodeWave<D, BN, PAGED>;
  __shared__ __attribute__((aligned(1024))) char tiles[4 * W::TILE];
  W st;
  st.kl[0] = (lds_char*)tiles;
  st.kl[1] = (lds_char*)tiles + W::TILE;
  st.vl[0] = (lds_char*)tiles + 2 * W::TILE;
  st.vl[1] = (lds_char*)tiles + 3 * W::TILE;
  const int bh = blockIdx.x / S, sp = blockIdx.x % S;
  if constexpr (PAGED) {
    // this sequence's valid length, at most what its block table can address
    const int b = bh / pc.H;
    st.head = bh % pc.H;
    st.H = pc.H;
    st.page_shift = pc.page_shift;
    st.num_pages = pc.num_pages;
    st.table = (const __attribute__((address_space(4))) int*)(pc.block_table + (size_t)b * pc.max_pages);
    st.kpool = K;
    st.vpool = V;
    const int len = __builtin_amdgcn_readfirstlane(pc.seq_lens[b]);
    Nk = max(0, min(len, pc.max_pages << pc.page_shift));
    const int per = (Nk + S - 1) / S;
    chunk = (per + BN - 1) / BN * BN;
  }
  st.Nq = Nq;
  st.Nk = Nk;
  st.causal = causal;
  st.c = c;
  st.lane = threadIdx.x;
  st.h = st.lane >> 5;
  st.l32 = st.lane & 31;
  st.qrow = st.l32;
  const int k_lo = sp * chunk;
  st.k_hi = min(Nk, k_lo + chunk);
  const size_t qhead = (size_t)bh * Nq * D, khead = PAGED ? 0 : (size_t)bh * Nk * D;

#pragma unroll
  for (int t = 0; t < W::KSTEPS; ++t) {
    i32x4 x = {0, 0, 0, 0};
    if (st.qrow < Nq) x = *(const i32x4*)(Q + qhead + (size_t)st.qrow * D + 16 * t + 8 * st.h);
    x ^= qsign;
    st.qf[t] = __builtin_bit_cast(bf16x8, x);
  }
#pragma unroll
  for (int db = 0; db < W::DBLK; ++db) st.oacc[db] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;

  if (k_lo < st.k_hi) {
    if constexpr (!PAGED) {
      st.kres = make_rsrc(K + khead, (uint32_t)Nk * D * 2);
      st.vres = make_rsrc(V + khead, (uint32_t)Nk * D * 2);
      st.kg = K + khead;
      st.vg = V + khead;
    }
#pragma unroll
    for (int u = 0; u < W::LOADS; ++u) {
      const int p = u * 64 + st.lane;
      const int row = p / W::DCH, pc = p % W::DCH;
      st.koff[u] = (row * D + (pc ^ bf16_swz_k<D>(row)) * 8) * 2;
      st.voff[u] = (row * D + (pc ^ bf16_swz_v<D>(row)) * 8) * 2;
    }
    const int t0 = k_lo / BN, t1 = (st.k_hi + BN - 1) / BN;
    if constexpr (PAGED) st.page_next = st.load_page(t0);
    st.template issue<0>(t0);
    int t = t0;
    for (; t + 1 < t1; t += 2) {
      st.template tile<0>(t);
      st.template tile<1>(t + 1);
    }
    if (t < t1) st.template tile<0>(t);
    wait_vmem();                     // no copy may land in LDS after the wave ends
  }

  // ---- partial: o_r = O / l (fp32), lse_r = ln 2 (m + log2 l); empty: 0, -inf
  const float lt = halves_sum(st.l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (st.qrow < Nq) {
    const long long prow = (long long)sp * rows + (long long)bh * Nq + st.qrow;
    float* orow = OP + prow * D;
#pragma unroll
    for (int db = 0; db < W::DBLK; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = st.oacc[db][4 * g4 + e] * inv;
        *(f32x4*)(orow + db * 32 + 8 * g4 + 4 * st.h) = y;
      }
    if (st.h == 0) {
      const float muse = st.m == -INFINITY ? 0.f : st.m;
      LP[prow] = lt > 0.f ? (muse + log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

}  // namespace

size_t decode_workspace_bytes(long long rows, int d, int splits) {
  return (size_t)splits * rows * ((size_t)d * 4 + 4);
}

int decode_chunk(int Nk, int d, int splits) {
  const int bn = d == 128 ? 32 : 64;
  const int per = (Nk + splits - 1) / splits;
  return (per + bn - 1) / bn * bn;
}

hipError_t launch_attn_decode(const DecodeArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.BH * a.Nq;
  float* op = (float*)a.workspace;
  float* lp = op + (size_t)a.splits * rows * a.d;
  const float c = fabsf(a.scale) * kLog2e;
  const int qsign = a.scale < 0.f ? (int)0x80008000u : 0;
  const dim3 grid((unsigned)((long long)a.BH * a.splits));
  const uint16_t* q = (const uint16_t*)a.q;
  const uint16_t* k = (const uint16_t*)a.k;
  const uint16_t* v = (const uint16_t*)a.v;
  if (a.block_table) {
    // paged: 32-key tiles at both head sizes (a tile never spans two pages)
    int shift = 0;
    while ((1 << shift) < a.page_size) ++shift;
    const PagedCache pc{a.block_table, a.seq_lens, a.H, a.num_pages, shift, a.max_pages};
    if (a.d == 128)
      hipLaunchKernelGGL((attn_decode_kernel<128, 32, true>), grid, dim3(64), 0, stream, q, k, v, op,
                         lp, a.Nq, 0, a.splits, 0, c, a.causal, qsign, rows, pc);
    else
      hipLaunchKernelGGL((attn_decode_kernel<64, 32, true>), grid, dim3(64), 0, stream, q, k, v, op,
                         lp, a.Nq, 0, a.splits, 0, c, a.causal, qsign, rows, pc);
  } else {
    const int chunk = decode_chunk(a.Nk, a.d, a.splits);
    const PagedCache none{nullptr, nullptr, 1, 0, 0, 0};
    if (a.d == 128)
      hipLaunchKernelGGL((attn_decode_kernel<128, 32, false>), grid, dim3(64), 0, stream, q, k, v, op,
                         lp, a.Nq, a.Nk, a.splits, chunk, c, a.causal, qsign, rows, none);
    else
      hipLaunchKernelGGL((attn_decode_kernel<64, 64, false>), grid, dim3(64), 0, stream, q, k, v, op,
                         lp, a.Nq, a.Nk, a.splits, chunk, c, a.causal, qsign, rows, none);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_lse_merge(op, lp, a.splits, rows, a.d, a.o, a.lse, stream);
}

}  // namespace mi355attn
