/*
 * attn.h - C ABI of the MI355X (gfx950) tiled attention forward library.
 *
 * The library computes the fused attention forward pass
 *
 *     O = softmax(scale * Q K^T + mask) V,   LSE = log sum exp(scale * Q K^T + mask)
 *
 * block by block with an online (running max / running sum) softmax, so the
 * N x N score matrix is never stored. Sources (web pages on FlashAttention-3,
 * cited by title and section):
 *   [WGC] "Warp Group Cluster 优化：Flash Attention V3 在 H100 上的 FP8 融合计算实践"
 *   [JJ]  "大模型加速-核心网络算子-Flash Attention V3"
 *   [YT]  "FlashAttention V3：优化框架吞吐量的关键技术实践"
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller. No call
 *     allocates, frees, copies to the host or synchronises. The library keeps
 *     no state between calls apart from a cache of device properties, and one
 *     static device buffer (ATTN_NOALLOC_SCRATCH_BYTES per device, part of its
 *     code object) that only attn_decode_noalloc uses.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL means
 *     the default stream) and the call returns before the work finishes.
 *     Device-side faults surface at the caller's next synchronisation.
 *   - Tensors are contiguous, row-major [B][H][N][d] (d fastest). bf16 is
 *     bfloat16 bits, fp8 is OCP E4M3FN bytes (bias 7, max 448, no inf).
 *   - Every argument is validated before any HIP call; a failed check
 *     returns a negative ATTN_E_* code and enqueues nothing.
 *   - B*H*N == 0 is a valid empty problem: nothing is launched and ATTN_OK is
 *     returned (tensor pointers are then not inspected).
 *   - Calls are thread-safe. Calls that overlap on one stream run in order;
 *     calls on different streams writing the same outputs race (caller's
 *     responsibility).
 */
#ifndef MI355_ATTN_H
#define MI355_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v for attn_fwd. o is always bf16, lse always fp32. */
typedef enum {
  ATTN_DTYPE_BF16 = 0,      /* q, k, v bf16; bf16 MFMA contractions                 */
  ATTN_DTYPE_FP8_E4M3 = 1,  /* q, k, v E4M3 codes with per-block descales; fp8 MFMA */
  ATTN_DTYPE_FP8_PV = 2     /* q, k bf16 (S = Q K^T on bf16 MFMAs); v E4M3 codes with
                               per-block descales, P in E4M3, O += P V on fp8 MFMAs  */
} attn_dtype;

/* Return codes. */
enum {
  ATTN_OK = 0,
  ATTN_E_NULL = -1,      /* a required pointer is NULL                               */
  ATTN_E_SHAPE = -2,     /* B, H or N negative or beyond the supported maximum        */
  ATTN_E_HEADDIM = -3,   /* d not supported by the call (64, 128; 256 where stated)   */
  ATTN_E_DTYPE = -4,     /* unknown dtype, or fp8 descale pointers missing            */
  ATTN_E_ALIGN = -5,     /* a tensor pointer is not 16-byte aligned (lse: 4-byte)     */
  ATTN_E_WINDOW = -6,    /* window < -1, or causal not 0/1                            */
  ATTN_E_ALIAS = -7,     /* an output overlaps an input or another output             */
  ATTN_E_LAUNCH = -8,    /* the kernel launch failed (no device, bad stream, ...)     */
  ATTN_E_SCALE = -9,     /* scale is not finite                                       */
  ATTN_E_WORKSPACE = -10,/* decode workspace NULL, misaligned or too small            */
  ATTN_E_SCRATCH = -11   /* attn_decode_noalloc: the call needs more than its scratch */
};

/* Largest supported sizes (index arithmetic is 64-bit; these bound the grid). */
/* Longest sequence: the byte offset of a tile past one head's K or V end
 * must stay inside the 32-bit range of the buffer descriptors the kernels
 * read through ((2^23 + 128) * 128 * 2 < 2^32). */
#define ATTN_MAX_N (1 << 23)
/* The same bound at d = 256, where a row is twice as long. */
#define ATTN_MAX_N_D256 (1 << 22)
#define ATTN_MAX_BH (1 << 24)
/* Rows per fp8 scaling block, for Q, K and V alike. */
#define ATTN_FP8_BLOCK_ROWS 128

/*
 * attn_fwd - fused attention forward.
 *
 * Computes, for every batch b, head h and query row i, over the allowed key
 * set A(i):
 *   s_ij = scale * <q_i, k_j>  (dtype 1: scale * dq * dk * <q8_i, k8_j>)
 *   o_i  = sum_{j in A(i)} softmax_j(s_i) * v_j    (dtypes 1, 2: v_j = v8_j * dv)
 *   lse_i = ln sum_{j in A(i)} exp(s_ij)           (natural log)
 * The tiled, online-softmax evaluation follows [WGC] section 2 (local max and
 * sum per key block, running statistics, rescale of the output) and [JJ]
 * section 2.4; the fused softmax + mask + matmul follows [YT] section 1.2.
 *
 *   q, k, v   [B][H][N][d]. Read only. dtype 0: all bf16; dtype 1: all E4M3
 *             bytes; dtype 2: q and k bf16, v E4M3 bytes.
 *   o         [B][H][N][d] bf16 output (fp32 accumulation, rounded to nearest
 *             even at the end: [WGC] section 3).
 *   lse       [B][H][N] fp32 output, may NOT be NULL.
 *   B, H, N   batch, heads, sequence length (queries = keys = N).
 *   d         head dimension: 64 or 128 ([WGC] "适用场景"); 256 with dtype 0
 *             ([WGC] "后续方向" lists it as the next step), with
 *             N <= ATTN_MAX_N_D256.
 *   causal    1: key j allowed only if j <= i. 0: no causal cut.
 *   window    -1: no window. w >= 0: keys with i - w <= j <= i (causal) or
 *             |i - j| <= w (non-causal): the band of [YT] section 2.1.2, both
 *             ends inclusive. Key tiles wholly outside the allowed set are
 *             skipped, never loaded ([YT] section 2.1.2).
 *   scale     finite multiplier of Q K^T (commonly 1/sqrt(d)); 0 and negative
 *             values are allowed.
 *   dtype     attn_dtype.
 *   descale_q, descale_k, descale_v
 *             fp32 [B][H][ceil(N/128)] dequantisation factors, one per 128-row
 *             block of the corresponding E4M3 tensor, as written by
 *             attn_fp8_quantize ([WGC] section 3, per-block scaling). dtype 1
 *             needs all three; dtype 2 needs descale_v only; the others are
 *             ignored and may be NULL. attn_fp8_quantize writes positive,
 *             normal, finite values (amax / 448, at least 2^-126; 1 for an
 *             all-zero block). Q and K
 *             descales enter the score scale as given. A V descale that is
 *             zero, subnormal, negative or not finite is applied as 2^-127:
 *             that block's keys still count in the softmax denominator, but
 *             their values add nothing to O.
 *   stream    hipStream_t or NULL.
 *
 * dtype 2 keeps the score contraction in bf16 and only P and V in E4M3 (the
 * FP8 GEMM of [JJ] section 2.3 for PV alone): on data whose large outlier
 * channels are shared by Q and K, E4M3 scores carry an error that grows with
 * |s|, and this mode removes it at the cost of bf16 speed for QK^T.
 * A row whose allowed set is empty (impossible with the masks above, since
 * j = i is always allowed) would get o = 0 and lse = -inf.
 * Returns ATTN_OK or an ATTN_E_* code.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int N, int d, int causal, int window, float scale,
             int dtype, const float* descale_q, const float* descale_k,
             const float* descale_v, void* stream);

/* Largest number of partial results attn_lse_merge accepts. */
#define ATTN_MAX_MERGE 4096

/*
 * attn_lse_merge - merge R partial results computed over disjoint key sets.
 *
 * For every row (b, h, i), partial r holds o_r, the softmax over its own key
 * set applied to V, and lse_r, the natural log of that set's softmax
 * denominator (as attn_fwd writes them). The merged row is
 *   lse = ln sum_r exp(lse_r)
 *   o   = sum_r exp(lse_r - lse) * o_r
 * the update of the running statistics and output of the online softmax
 * ([WGC] section 2) taken across partial results, which a split of the keys
 * over workgroups or devices needs ([YT] section 2.3.1). Partials with
 * lse_r = -inf carry no weight; a row whose partials are all -inf gets o = 0
 * and lse = -inf. Inputs holding NaN or +inf give undefined rows.
 *
 *   o_part    fp32 [R][B][H][N][d], read only.
 *   lse_part  fp32 [R][B][H][N], read only.
 *   o         bf16 [B][H][N][d] output (fp32 sums, rounded to nearest even).
 *   lse       fp32 [B][H][N] output.
 *   R         number of partials, 1 .. ATTN_MAX_MERGE.
 *   d         64, 128 or 256.
 *   stream    hipStream_t or NULL. The call only enqueues one kernel.
 * All pointers are device pointers owned by the caller; tensors 16-byte
 * aligned, fp32 LSE arrays 4-byte aligned. Outputs may not overlap inputs or
 * each other. B*H*N = 0 is an empty problem (ATTN_OK, nothing enqueued).
 * Returns ATTN_OK or an ATTN_E_* code.
 */
int attn_lse_merge(const float* o_part, const float* lse_part, void* o, float* lse,
                   int R, int B, int H, int N, int d, void* stream);

/* Most queries per (batch, head) attn_decode takes: one 32-wide MFMA block. */
#define ATTN_MAX_DECODE_Q 32

/*
 * attn_decode_workspace_bytes - device workspace attn_decode needs:
 * splits * B * H * Nq * (4 d + 4) bytes (the fp32 partial outputs and their
 * log-sum-exps). Returns 0 for arguments attn_decode would reject.
 */
size_t attn_decode_workspace_bytes(int B, int H, int Nq, int d, int splits);

/*
 * attn_decode - attention of Nq <= 32 new queries against Nk >= Nq cached
 * keys and values of the same sequences (decoding with a key/value cache,
 * [JJ] section 3). The queries are the last Nq positions: query i sits at
 * position Nk - Nq + i and, with causal = 1, attends keys j <= Nk - Nq + i.
 *   s_ij = scale * <q_i, k_j>;  o_i = sum_j softmax_j(s_i) v_j;
 *   lse_i = ln sum_j exp(s_ij)
 * The keys of every (b, h) are split into `splits` contiguous chunks of
 * ceil(Nk / splits) keys (rounded up to the 32- or 64-key tile); each chunk's
 * tiled online softmax ([WGC] sections 1-2) writes an fp32 partial into the
 * workspace, and the partials are merged as attn_lse_merge does. Two kernels
 * on `stream`; nothing is allocated.
 *
 *   q         bf16 [B][H][Nq][d]; k, v bf16 [B][H][Nk][d]. Read only.
 *   o         bf16 [B][H][Nq][d] output; lse fp32 [B][H][Nq] output.
 *   Nq        1 .. ATTN_MAX_DECODE_Q (0: empty problem); Nk: Nq .. ATTN_MAX_N.
 *   d         64 or 128.
 *   causal    0 or 1 (bottom-right aligned, as above).
 *   scale     finite; 0 and negative allowed.
 *   splits    1 .. ATTN_MAX_MERGE key chunks per (b, h); more chunks give more
 *             workgroups (B * H * splits) for small batches.
 *   workspace device memory of at least attn_decode_workspace_bytes(B, H, Nq,
 *             d, splits) bytes, 16-byte aligned, owned by the caller; its
 *             contents are scratch.
 * Pointers are device pointers owned by the caller; tensors 16-byte aligned,
 * lse 4-byte aligned; outputs and workspace may not overlap inputs or each
 * other. Returns ATTN_OK or an ATTN_E_* code (ATTN_E_WORKSPACE: workspace
 * NULL, misaligned or too small).
 */
int attn_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int Nq, int Nk, int d, int causal, float scale, int splits,
                void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the static scratch buffer attn_decode_noalloc uses (per device). */
#define ATTN_NOALLOC_SCRATCH_BYTES (16 << 20)

/*
 * attn_decode_noalloc - attn_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. It computes exactly what attn_decode computes, with the
 * same kernels, but keeps the fp32 partials and log-sum-exps in a static
 * buffer of ATTN_NOALLOC_SCRATCH_BYTES bytes that the library holds on every
 * device it runs on, from the load of its code object until the process
 * ends. The call allocates and frees nothing.
 *
 *   All arguments as in attn_decode, without workspace and workspace_bytes.
 *   The work uses the buffer of the device `stream` belongs to (the current
 *   device for the NULL stream).
 * The buffer needs no clearing (every slot a call reads it has written
 * first). Calls on one device share that device's buffer: calls that overlap
 * on one device (different streams or host threads without ordering) race
 * on it; calls ordered on one stream are safe. Returns ATTN_OK or an ATTN_E_*
 * code: ATTN_E_SCRATCH when attn_decode_workspace_bytes(B, H, Nq, d, splits)
 * exceeds ATTN_NOALLOC_SCRATCH_BYTES (nothing is enqueued; fewer splits or a
 * smaller batch per call fit), ATTN_E_LAUNCH if the buffer's device address
 * cannot be obtained or the launch fails.
 */
int attn_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int Nq, int Nk, int d, int causal, float scale, int splits,
                        void* stream);

/* Page sizes (positions per page) attn_decode_paged takes: powers of two in
 * this range, so a 32-key tile never spans two pages. */
#define ATTN_MIN_PAGE 32
#define ATTN_MAX_PAGE 4096

/*
 * attn_decode_paged - attn_decode against a paged key/value cache (the
 * PagedAttention cache management that [WGC] "limitations and follow-up
 * directions" names as a next step). Sequence b's cached positions live in
 * pages of page_size positions scattered over a shared pool; position p of
 * sequence b is row p % page_size of page block_table[b][p / page_size].
 * Sequence b holds seq_lens[b] valid positions, and its Nq queries are its
 * last Nq positions (query i at seq_lens[b] - Nq + i, causal as in
 * attn_decode). Per (b, h) the result is attn_decode's over the gathered
 * seq_lens[b] positions; each sequence's keys are split into `splits` chunks
 * of its own length. Two kernels on `stream`; nothing is allocated; no host
 * synchronisation (block_table and seq_lens are read on the device).
 *
 *   q            bf16 [B][H][Nq][d]. Read only.
 *   k_cache,
 *   v_cache      bf16 pools [num_pages][H][page_size][d] (one page holds every
 *                head's rows for its positions). Read only.
 *   block_table  int32 [B][max_pages], device memory: physical page of each
 *                logical page. Entries past a sequence's last page are unused.
 *   seq_lens     int32 [B], device memory: valid positions per sequence; the
 *                caller keeps Nq <= seq_lens[b] <= max_pages * page_size.
 *   o, lse       outputs as in attn_decode.
 *   Nq           1 .. ATTN_MAX_DECODE_Q (0: empty problem); d: 64 or 128.
 *   num_pages    pages in each pool (>= 1); page_size: a power of two in
 *                [ATTN_MIN_PAGE, ATTN_MAX_PAGE]; max_pages >= 1 with
 *                max_pages * page_size <= ATTN_MAX_N.
 *   causal, scale, splits, workspace, workspace_bytes: as in attn_decode
 *                (workspace size from attn_decode_workspace_bytes).
 * Device-side values outside the contract cannot make the kernel access
 * memory outside the pools, the table row or the outputs: a table entry
 * outside [0, num_pages) reads as a page of zeros, seq_lens[b] is clamped to
 * [0, max_pages * page_size], and rows past seq_lens[b] are never read. The
 * results for such inputs are unspecified; seq_lens[b] = 0 gives o = 0,
 * lse = -inf. Pointers are device pointers owned by the caller; tensors
 * 16-byte aligned, lse, block_table and seq_lens 4-byte aligned; outputs and
 * workspace may not overlap inputs or each other. Returns ATTN_OK or an
 * ATTN_E_* code.
 */
int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                      const int* block_table, const int* seq_lens, void* o, float* lse,
                      int B, int H, int Nq, int d, int num_pages, int page_size, int max_pages,
                      int causal, float scale, int splits, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * attn_fp8_quantize - bf16 -> E4M3 with one scaling factor per 128-row block.
 *
 * For each (b, h) and each block of 128 rows (the last block may be shorter):
 *   amax = max |x| over the block (per_tensor = 1: over the whole tensor)
 *   r = fp32(448 / amax), descale = fp32(amax / 448); amax == 0 gives r = 1,
 *   descale = 1; 0 < amax < 448 * 2^-126 (where amax / 448 would not be a
 *   normal fp32) gives descale = 2^-126 and r = 2^126, its exact reciprocal
 *   x8 = E4M3(fp32(x * r)), round to nearest even, saturating at +-448
 * So every descale is a positive, normal, finite fp32 value and a zero
 * element always encodes as 0.
 * [WGC] section 3 (dynamic per-block scaling into the range of max 448, fp32
 * accumulation downstream); the format is [JJ] section 1.5's E4M3.
 *
 *   x_bf16    [B][H][N][d] bf16 input. Read only.
 *   x_fp8     [B][H][N][d] E4M3 output bytes.
 *   descale   [B][H][ceil(N/128)] fp32 output.
 *   d         64 or 128.
 *   per_tensor 0: per-block amax. 1: one amax for the whole tensor, written
 *             into every descale slot (the naive baseline), so attn_fwd treats
 *             both modes alike.
 * The per-tensor mode runs three kernels on `stream` and uses `descale` as its
 * only scratch; nothing else is allocated. Inputs holding Inf or NaN give
 * undefined codes. Returns ATTN_OK or an ATTN_E_* code.
 */
int attn_fp8_quantize(const void* x_bf16, void* x_fp8, float* descale,
                      int B, int H, int N, int d, int per_tensor, void* stream);

/*
 * attn_fp8_quantize_rotated - attn_fp8_quantize of the rotated tensor: the
 * incoherent processing that [JJ] (introduction, contribution 3, and section
 * 3's summary) pairs with FP8 block quantisation. Every row x (d values) is
 * first replaced by
 *   x' = (x * s) H / sqrt(d)
 * with H the d x d Sylvester Hadamard matrix (H_1 = [1], H_2n = [[H_n, H_n],
 * [H_n, -H_n]]) and s the caller's signs; then x' is quantised exactly as
 * attn_fp8_quantize quantises x (per 128-row block or per tensor). The matrix
 * diag(s) H / sqrt(d) is orthogonal, so quantising Q and K with the SAME signs
 * and passing the codes and descales to attn_fwd (dtype 1) computes the same
 * attention: (Q M)(K M)^T = Q K^T. Channels that are large in both Q and K
 * are spread over all d channels, which lowers the E4M3 score error. V is
 * quantised with attn_fp8_quantize, unrotated.
 * The rotation is computed in fp32 in this order (its values decide the
 * codes): sign flips; the fast Walsh-Hadamard butterfly with stages
 * h = 1, 2, 4, ..., d/2, where for every j with bit h clear x[j] becomes
 * x[j] + x[j+h] and x[j+h] becomes x[j] - x[j+h] (one fp32 rounding each);
 * one fp32 multiply by fp32(1/sqrt(d)).
 *
 *   signs     int8 [d] device memory, 8-byte aligned, read only: entry c < 0
 *             means s_c = -1, any other value s_c = +1. Draw them at random
 *             once and use them for both Q and K.
 *   other arguments as in attn_fp8_quantize (d = 64 or 128).
 * Returns ATTN_OK or an ATTN_E_* code (ATTN_E_NULL for NULL signs).
 */
int attn_fp8_quantize_rotated(const void* x_bf16, void* x_fp8, float* descale,
                              const signed char* signs, int B, int H, int N, int d,
                              int per_tensor, void* stream);

/* Static, human-readable text for a return code (never NULL). */
const char* attn_strerror(int code);

/* Library version as major * 10000 + minor * 100 + patch. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MI355_ATTN_H */
