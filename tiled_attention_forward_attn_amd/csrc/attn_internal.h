// Internal declarations shared by the HIP translation units of the library.
// Not part of the public ABI (that is include/attn.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355attn {

// Launch parameters common to the attention kernels, validated by the C ABI.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const float* dq;   // fp8 descales (nullptr for bf16)
  const float* dk;
  const float* dv;
  int BH;            // B * H
  int N;
  int d;
  int causal;
  int window;
  float scale;
};

// Decode launch parameters, validated by the C ABI.
struct DecodeArgs {
  const void* q;     // bf16 [BH][Nq][d]
  const void* k;     // bf16 [BH][Nk][d], or the paged pool [num_pages][H][page_size][d]
  const void* v;
  void* o;           // bf16 [BH][Nq][d]
  float* lse;        // [BH][Nq]
  void* workspace;   // fp32 partials [splits][BH * Nq][d], then lse [splits][BH * Nq]
  int BH, Nq, Nk, d, causal, splits;
  float scale;
  // paged cache (block_table == nullptr: contiguous k, v)
  const int* block_table = nullptr;   // [B][max_pages]
  const int* seq_lens = nullptr;      // [B]
  int H = 1, num_pages = 0, page_size = 0, max_pages = 0;
};

hipError_t launch_attn_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_attn_decode(const DecodeArgs& a, hipStream_t stream);
size_t decode_workspace_bytes(long long rows, int d, int splits);
// Keys per split: ceil(Nk / splits) rounded up to the key tile.
int decode_chunk(int Nk, int d, int splits);
// qk_bf16: q and k are bf16 (S = Q K^T on bf16 MFMAs), v stays E4M3.
hipError_t launch_attn_fwd_fp8(const FwdArgs& a, bool qk_bf16, hipStream_t stream);
// rows = B * H * N; d in {64, 128, 256}.
hipError_t launch_lse_merge(const float* o_part, const float* lse_part, int R, long long rows, int d,
                            void* o, float* lse, hipStream_t stream);
// signs: nullptr for the plain quantiser; else d signs of the rotation
// (incoherent processing) applied to every row first.
hipError_t launch_fp8_quantize(const void* x, void* x8, float* descale, const int8_t* signs, int BH,
                               int N, int d, int per_tensor, hipStream_t stream);

}  // namespace mi355attn
