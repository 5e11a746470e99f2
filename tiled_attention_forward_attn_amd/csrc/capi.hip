// C ABI of the attention library: argument validation and kernel dispatch.
// Every check runs before the first HIP call, so all error paths are testable
// on a machine without a GPU. See include/attn.h for the contract.
#include "attn.h"
#include "attn_internal.h"

#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

using namespace mi355attn;

namespace {

constexpr int kVersion = 1 * 10000 + 7 * 100 + 0;
constexpr long long kMaxGrid = 2147483647LL;  // gridDim.x limit

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

bool aligned(const void* p, uintptr_t n) { return ((uintptr_t)p % n) == 0; }

// Shape checks shared by attn_fwd and attn_fp8_quantize; *empty is set for
// B*H*N == 0. d = 256 only where d256 is set (the bf16 path).
int check_shape(int B, int H, int N, int d, bool d256, bool* empty) {
  if (B < 0 || H < 0 || N < 0) return ATTN_E_SHAPE;
  *empty = (long long)B * H * N == 0;
  if (*empty) return ATTN_OK;
  if (N > ATTN_MAX_N || (long long)B * H > ATTN_MAX_BH) return ATTN_E_SHAPE;
  if (d != 64 && d != 128 && !(d256 && d == 256)) return ATTN_E_HEADDIM;
  if (d == 256 && N > ATTN_MAX_N_D256) return ATTN_E_SHAPE;
  // one workgroup per 128-row block of every head must fit the 1-D grid
  if ((long long)((N + 127) / 128) * B * H > kMaxGrid) return ATTN_E_SHAPE;
  return ATTN_OK;
}

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int N, int d, int causal, int window, float scale,
                        int dtype, const float* descale_q, const float* descale_k,
                        const float* descale_v, void* stream) {
  bool empty = false;
  int rc = check_shape(B, H, N, d, dtype == ATTN_DTYPE_BF16, &empty);
  if (rc != ATTN_OK || empty) return rc;
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_FP8_E4M3 && dtype != ATTN_DTYPE_FP8_PV)
    return ATTN_E_DTYPE;
  if (!q || !k || !v || !o || !lse) return ATTN_E_NULL;
  const bool fp8 = dtype == ATTN_DTYPE_FP8_E4M3;   // all E4M3
  const bool pv8 = dtype == ATTN_DTYPE_FP8_PV;     // q, k bf16; v E4M3
  if (fp8 && (!descale_q || !descale_k || !descale_v)) return ATTN_E_NULL;
  if (pv8 && !descale_v) return ATTN_E_NULL;
  if (causal != 0 && causal != 1) return ATTN_E_WINDOW;
  if (window < -1) return ATTN_E_WINDOW;
  if (!isfinite(scale)) return ATTN_E_SCALE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return ATTN_E_ALIGN;
  if (fp8 && (!aligned(descale_q, 4) || !aligned(descale_k, 4))) return ATTN_E_ALIGN;
  if ((fp8 || pv8) && !aligned(descale_v, 4)) return ATTN_E_ALIGN;

  const size_t elems = (size_t)B * H * N * d;
  const size_t qk_bytes = elems * (fp8 ? 1 : 2);
  const size_t v_bytes = elems * (fp8 || pv8 ? 1 : 2);
  const size_t o_bytes = elems * 2;
  const size_t lse_bytes = (size_t)B * H * N * sizeof(float);
  const void* ins[3] = {q, k, v};
  const size_t in_bytes[3] = {qk_bytes, qk_bytes, v_bytes};
  for (int i = 0; i < 3; ++i) {
    if (overlap(o, o_bytes, ins[i], in_bytes[i]) || overlap(lse, lse_bytes, ins[i], in_bytes[i]))
      return ATTN_E_ALIAS;
  }
  if (overlap(o, o_bytes, lse, lse_bytes)) return ATTN_E_ALIAS;
  if (fp8 || pv8) {
    const size_t ds_bytes = (size_t)B * H * ((N + ATTN_FP8_BLOCK_ROWS - 1) / ATTN_FP8_BLOCK_ROWS) * sizeof(float);
    const void* dss[3] = {fp8 ? descale_q : nullptr, fp8 ? descale_k : nullptr, descale_v};
    for (const void* ds : dss)
      if (ds && (overlap(o, o_bytes, ds, ds_bytes) || overlap(lse, lse_bytes, ds, ds_bytes)))
        return ATTN_E_ALIAS;
  }

  FwdArgs a{q, k, v, o, lse, fp8 ? descale_q : nullptr, fp8 ? descale_k : nullptr,
            (fp8 || pv8) ? descale_v : nullptr, B * H, N, d, causal, window, scale};
  const hipError_t e = (fp8 || pv8) ? launch_attn_fwd_fp8(a, pv8, (hipStream_t)stream)
                                    : launch_attn_fwd_bf16(a, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

namespace {

// attn_fp8_quantize and attn_fp8_quantize_rotated (signs != nullptr).
int quantize_call(const void* x_bf16, void* x_fp8, float* descale, const signed char* signs,
                  bool rotated, int B, int H, int N, int d, int per_tensor, void* stream) {
  bool empty = false;
  int rc = check_shape(B, H, N, d, false, &empty);
  if (rc != ATTN_OK || empty) return rc;
  if (!x_bf16 || !x_fp8 || !descale || (rotated && !signs)) return ATTN_E_NULL;
  if (per_tensor != 0 && per_tensor != 1) return ATTN_E_DTYPE;
  if (!aligned(x_bf16, 16) || !aligned(x_fp8, 8) || !aligned(descale, 4) ||
      (rotated && !aligned(signs, 8)))
    return ATTN_E_ALIGN;
  const size_t elems = (size_t)B * H * N * d;
  const size_t ds_bytes = (size_t)B * H * ((N + ATTN_FP8_BLOCK_ROWS - 1) / ATTN_FP8_BLOCK_ROWS) * sizeof(float);
  if (overlap(x_fp8, elems, x_bf16, elems * 2) || overlap(descale, ds_bytes, x_bf16, elems * 2) ||
      overlap(descale, ds_bytes, x_fp8, elems))
    return ATTN_E_ALIAS;
  if (rotated && (overlap(x_fp8, elems, signs, d) || overlap(descale, ds_bytes, signs, d)))
    return ATTN_E_ALIAS;
  const hipError_t e = launch_fp8_quantize(x_bf16, x_fp8, descale, (const int8_t*)signs, B * H, N, d,
                                           per_tensor, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

}  // namespace

extern "C" int attn_fp8_quantize(const void* x_bf16, void* x_fp8, float* descale, int B, int H,
                                 int N, int d, int per_tensor, void* stream) {
  return quantize_call(x_bf16, x_fp8, descale, nullptr, false, B, H, N, d, per_tensor, stream);
}

extern "C" int attn_fp8_quantize_rotated(const void* x_bf16, void* x_fp8, float* descale,
                                         const signed char* signs, int B, int H, int N, int d,
                                         int per_tensor, void* stream) {
  return quantize_call(x_bf16, x_fp8, descale, signs, true, B, H, N, d, per_tensor, stream);
}

extern "C" int attn_lse_merge(const float* o_part, const float* lse_part, void* o, float* lse,
                              int R, int B, int H, int N, int d, void* stream) {
  if (B < 0 || H < 0 || N < 0 || R < 1 || R > ATTN_MAX_MERGE) return ATTN_E_SHAPE;
  const long long rows = (long long)B * H * N;
  if (rows == 0) return ATTN_OK;
  if ((long long)B * H > ATTN_MAX_BH || N > ATTN_MAX_N) return ATTN_E_SHAPE;
  if (d != 64 && d != 128 && d != 256) return ATTN_E_HEADDIM;
  // one workgroup per 256 / (d / 4) rows must fit the 1-D grid
  if ((rows + 256 / (d / 4) - 1) / (256 / (d / 4)) > kMaxGrid) return ATTN_E_SHAPE;
  if (!o_part || !lse_part || !o || !lse) return ATTN_E_NULL;
  if (!aligned(o_part, 16) || !aligned(o, 16) || !aligned(lse_part, 4) || !aligned(lse, 4))
    return ATTN_E_ALIGN;
  const size_t op_bytes = (size_t)R * rows * d * sizeof(float);
  const size_t lp_bytes = (size_t)R * rows * sizeof(float);
  const size_t o_bytes = (size_t)rows * d * 2;
  const size_t lse_bytes = (size_t)rows * sizeof(float);
  if (overlap(o, o_bytes, o_part, op_bytes) || overlap(o, o_bytes, lse_part, lp_bytes) ||
      overlap(lse, lse_bytes, o_part, op_bytes) || overlap(lse, lse_bytes, lse_part, lp_bytes) ||
      overlap(o, o_bytes, lse, lse_bytes))
    return ATTN_E_ALIAS;
  const hipError_t e = launch_lse_merge(o_part, lse_part, R, rows, d, o, lse, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

namespace {

// Shape checks of attn_decode; *empty is set for B*H*Nq == 0.
int check_decode(int B, int H, int Nq, int Nk, int d, int splits, bool* empty) {
  if (B < 0 || H < 0 || Nq < 0 || Nq > ATTN_MAX_DECODE_Q || Nk < Nq || Nk > ATTN_MAX_N ||
      splits < 1 || splits > ATTN_MAX_MERGE)
    return ATTN_E_SHAPE;
  *empty = (long long)B * H * Nq == 0;
  if (*empty) return ATTN_OK;
  if ((long long)B * H > ATTN_MAX_BH) return ATTN_E_SHAPE;
  if (d != 64 && d != 128) return ATTN_E_HEADDIM;
  if ((long long)B * H * splits > kMaxGrid) return ATTN_E_SHAPE;
  return ATTN_OK;
}

}  // namespace

extern "C" size_t attn_decode_workspace_bytes(int B, int H, int Nq, int d, int splits) {
  bool empty = false;
  if (check_decode(B, H, Nq, Nq, d, splits, &empty) != ATTN_OK || empty) return 0;
  return decode_workspace_bytes((long long)B * H * Nq, d, splits);
}

namespace {

// The checks of attn_decode that do not involve the workspace: sizes, null
// pointers, flags, alignment, and outputs overlapping inputs or each other.
// *need is the workspace the call needs; *empty is set for an empty problem.
int check_decode_call(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int Nq, int Nk, int d, int causal, float scale, int splits,
                      size_t* need, bool* empty) {
  int rc = check_decode(B, H, Nq, Nk, d, splits, empty);
  if (rc != ATTN_OK || *empty) return rc;
  if (!q || !k || !v || !o || !lse) return ATTN_E_NULL;
  if (causal != 0 && causal != 1) return ATTN_E_WINDOW;
  if (!isfinite(scale)) return ATTN_E_SCALE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return ATTN_E_ALIGN;
  const long long rows = (long long)B * H * Nq;
  *need = decode_workspace_bytes(rows, d, splits);
  const size_t q_bytes = (size_t)rows * d * 2;
  const size_t kv_bytes = (size_t)B * H * Nk * d * 2;
  const size_t lse_bytes = (size_t)rows * sizeof(float);
  const void* ins[3] = {q, k, v};
  const size_t in_bytes[3] = {q_bytes, kv_bytes, kv_bytes};
  for (int i = 0; i < 3; ++i)
    if (overlap(o, q_bytes, ins[i], in_bytes[i]) || overlap(lse, lse_bytes, ins[i], in_bytes[i]))
      return ATTN_E_ALIAS;
  if (overlap(o, q_bytes, lse, lse_bytes)) return ATTN_E_ALIAS;
  return ATTN_OK;
}

}  // namespace

extern "C" int attn_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Nq, int Nk, int d, int causal, float scale,
                           int splits, void* workspace, size_t workspace_bytes, void* stream) {
  bool empty = false;
  size_t need = 0;
  int rc = check_decode_call(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, splits, &need, &empty);
  if (rc != ATTN_OK || empty) return rc;
  if (!workspace || !aligned(workspace, 16) || workspace_bytes < need) return ATTN_E_WORKSPACE;
  const long long rows = (long long)B * H * Nq;
  const size_t q_bytes = (size_t)rows * d * 2;
  const size_t kv_bytes = (size_t)B * H * Nk * d * 2;
  const size_t lse_bytes = (size_t)rows * sizeof(float);
  if (overlap(workspace, need, q, q_bytes) || overlap(workspace, need, k, kv_bytes) ||
      overlap(workspace, need, v, kv_bytes) || overlap(o, q_bytes, workspace, need) ||
      overlap(lse, lse_bytes, workspace, need))
    return ATTN_E_ALIAS;
  DecodeArgs a{q, k, v, o, lse, workspace, B * H, Nq, Nk, d, causal, splits, scale};
  const hipError_t e = launch_attn_decode(a, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

// ---- attn_decode_noalloc: attn_decode with the library's own scratch.
//
// The fp32 partials and log-sum-exps live in this array instead of a
// caller's workspace. Each device the library runs on holds its own copy from
// the moment the code object is loaded until the process ends. In host code
// the name `scratch` is only a host-side stand-in; the kernels get the
// address of the copy on the launch stream's device, looked up once per
// device with that device current and kept in g_scratch. The decode kernel writes every partial slot
// of a call (an empty key chunk writes o = 0, lse = -inf) before the merge
// reads it, so nothing needs clearing between calls.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the copy of `scratch` on the device `stream` belongs to
// (the current device for the NULL stream), looked up once per device with
// that device current; nullptr if the device cannot be determined.
void* scratch_for_stream(hipStream_t stream) {
  int dev = -1;
  if (stream ? hipStreamGetDevice(stream, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess)
    return nullptr;
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return nullptr;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" int attn_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                   int B, int H, int Nq, int Nk, int d, int causal, float scale,
                                   int splits, void* stream) {
  bool empty = false;
  size_t need = 0;
  int rc = check_decode_call(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, splits, &need, &empty);
  if (rc != ATTN_OK || empty) return rc;
  if (need > (size_t)ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_E_SCRATCH;
  void* ws = scratch_for_stream((hipStream_t)stream);
  if (!ws) return ATTN_E_LAUNCH;
  DecodeArgs a{q, k, v, o, lse, ws, B * H, Nq, Nk, d, causal, splits, scale};
  const hipError_t e = launch_attn_decode(a, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

extern "C" int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                                 const int* block_table, const int* seq_lens, void* o, float* lse,
                                 int B, int H, int Nq, int d, int num_pages, int page_size,
                                 int max_pages, int causal, float scale, int splits,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  bool empty = false;
  int rc = check_decode(B, H, Nq, Nq, d, splits, &empty);
  if (rc != ATTN_OK || empty) return rc;
  if (page_size < ATTN_MIN_PAGE || page_size > ATTN_MAX_PAGE || (page_size & (page_size - 1)) ||
      num_pages < 1 || max_pages < 1 || (long long)max_pages * page_size > ATTN_MAX_N ||
      (long long)num_pages * H * page_size > (1LL << 40))
    return ATTN_E_SHAPE;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !o || !lse) return ATTN_E_NULL;
  if (causal != 0 && causal != 1) return ATTN_E_WINDOW;
  if (!isfinite(scale)) return ATTN_E_SCALE;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(block_table, 4) || !aligned(seq_lens, 4))
    return ATTN_E_ALIGN;
  const long long rows = (long long)B * H * Nq;
  const size_t need = decode_workspace_bytes(rows, d, splits);
  if (!workspace || !aligned(workspace, 16) || workspace_bytes < need) return ATTN_E_WORKSPACE;
  const size_t q_bytes = (size_t)rows * d * 2;
  const size_t pool_bytes = (size_t)num_pages * H * page_size * d * 2;
  const size_t lse_bytes = (size_t)rows * sizeof(float);
  const void* ins[5] = {q, k_cache, v_cache, block_table, seq_lens};
  const size_t in_bytes[5] = {q_bytes, pool_bytes, pool_bytes,
                              (size_t)B * max_pages * sizeof(int), (size_t)B * sizeof(int)};
  for (int i = 0; i < 5; ++i) {
    if (overlap(o, q_bytes, ins[i], in_bytes[i]) || overlap(lse, lse_bytes, ins[i], in_bytes[i]) ||
        overlap(workspace, need, ins[i], in_bytes[i]))
      return ATTN_E_ALIAS;
  }
  if (overlap(o, q_bytes, lse, lse_bytes) || overlap(o, q_bytes, workspace, need) ||
      overlap(lse, lse_bytes, workspace, need))
    return ATTN_E_ALIAS;
  DecodeArgs a{q, k_cache, v_cache, o, lse, workspace, B * H, Nq, 0, d, causal, splits, scale};
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.H = H;
  a.num_pages = num_pages;
  a.page_size = page_size;
  a.max_pages = max_pages;
  const hipError_t e = launch_attn_decode(a, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

extern "C" const char* attn_strerror(int code) {
  switch (code) {
    case ATTN_OK: return "success";
    case ATTN_E_NULL: return "a required pointer is NULL";
    case ATTN_E_SHAPE: return "a size (B, H, N, Nq, Nk, R, splits, page_size, num_pages, max_pages) is out of range";
    case ATTN_E_HEADDIM: return "head dimension d not supported here (64 or 128; 256 for bf16 attn_fwd and attn_lse_merge)";
    case ATTN_E_DTYPE: return "unknown dtype or quantisation mode";
    case ATTN_E_ALIGN: return "a tensor pointer is misaligned (16 bytes for tensors, 4 for fp32 arrays)";
    case ATTN_E_WINDOW: return "causal must be 0 or 1 and window must be >= -1";
    case ATTN_E_ALIAS: return "an output buffer overlaps an input or another output";
    case ATTN_E_LAUNCH: return "kernel launch failed (no usable GPU or invalid stream)";
    case ATTN_E_SCALE: return "scale must be finite";
    case ATTN_E_WORKSPACE: return "decode workspace is NULL, misaligned or smaller than attn_decode_workspace_bytes";
    case ATTN_E_SCRATCH: return "attn_decode_noalloc needs more scratch than its static buffer holds (ATTN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown error code";
  }
}

extern "C" int attn_version(void) { return kVersion; }
