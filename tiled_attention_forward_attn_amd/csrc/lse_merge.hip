// Merge of R partial attention results over disjoint key sets, for gfx950.
//
// Partial r of a query row was computed over its own key set: o_r is the
// softmax over that set applied to V, lse_r the natural log of its softmax
// denominator. The merged row is
//   lse = ln sum_r exp(lse_r),   o = sum_r exp(lse_r - lse) o_r,
// with the largest lse_r subtracted before exponentiating; partials with
// lse_r = -inf carry no weight, and a row whose partials are all empty gets
// o = 0, lse = -inf. This is the running-statistics update and output rescale
// of the online softmax ([WGC] section 2) taken across partial results: the
// combination that a split of the keys over workgroups or devices needs
// ([WGC] limitations on sequence parallelism; [YT] section 2.3.1).
//
// HBM-bound: a row reads R (4 d + 4) bytes and writes 2 d + 4. D/4 lanes own
// a row, 4 consecutive columns each (16-byte loads, 8-byte bf16 stores), so a
// wave reads whole 256..1024-byte rows of one partial at a time; the loop
// over partials is unrolled so several of those loads are in flight. Every
// byte is read or written once, so the accesses carry the nontemporal hint.
#include "attn_device.h"
#include "attn_internal.h"

namespace mi355attn {
namespace {

constexpr int kMergeThreads = 256;

template <int D>
__global__ __launch_bounds__(kMergeThreads)
void lse_merge_kernel(const float* __restrict__ op, const float* __restrict__ lp, int R,
                      long long rows, uint16_t* __restrict__ o, float* __restrict__ lse) {
  constexpr int TPR = D / 4;                    // lanes per row
  constexpr int RPB = kMergeThreads / TPR;      // rows per workgroup
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = (threadIdx.x % TPR) * 4;
  if (row >= rows) return;

  float m = -INFINITY;
  for (int r = 0; r < R; ++r) m = fmaxf(m, lp[(long long)r * rows + row]);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float total = 0.f;
  if (m != -INFINITY) {
#pragma unroll 4
    for (int r = 0; r < R; ++r) {
      const long long pr = (long long)r * rows + row;
      const float w = expf(lp[pr] - m);          // 0 for an empty partial
      const f32x4 x = __builtin_nontemporal_load((const f32x4*)(op + pr * D + c));
      total += w;
      acc += w * x;
    }
  }
  const float inv = total > 0.f ? 1.f / total : 0.f;
  bf16x4 y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = (__bf16)(acc[e] * inv);
  __builtin_nontemporal_store(y, (bf16x4*)(o + row * D + c));
  if (c == 0) lse[row] = total > 0.f ? m + logf(total) : -INFINITY;
}

template <int D>
hipError_t launch_d(const float* op, const float* lp, int R, long long rows, uint16_t* o,
                    float* lse, hipStream_t s) {
  constexpr int RPB = kMergeThreads / (D / 4);
  const long long blocks = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL(lse_merge_kernel<D>, dim3((unsigned)blocks), dim3(kMergeThreads), 0, s, op, lp,
                     R, rows, o, lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_merge(const float* o_part, const float* lse_part, int R, long long rows, int d,
                            void* o, float* lse, hipStream_t stream) {
  uint16_t* ob = (uint16_t*)o;
  if (d == 64) return launch_d<64>(o_part, lse_part, R, rows, ob, lse, stream);
  if (d == 128) return launch_d<128>(o_part, lse_part, R, rows, ob, lse, stream);
  return launch_d<256>(o_part, lse_part, R, rows, ob, lse, stream);
}

}  // namespace mi355attn
