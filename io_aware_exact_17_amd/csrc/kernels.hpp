// kernels.hpp — host-side launch interface between the C ABI (api.cpp) and the
// HIP kernels.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Nq, Nk, d;
  float scale;
  int causal;
  hipStream_t stream;
  // Packed variable-length batch (null for the dense [B, H, N, d] layout):
  // q, o [total_q, H, d], k, v [total_k, H, d], lse [H, total_q]; sequence b
  // owns query rows cu_q[b] .. cu_q[b+1]-1 and key rows cu_k[b] .. cu_k[b+1]-1;
  // Nq is then the longest query length (it sizes the grid).
  const int32_t* cu_q = nullptr;
  const int32_t* cu_k = nullptr;
  int total_q = 0;
  // Block-sparse mask (d = 128, dense layout): uint8 [H, nqb, nkb] over
  // 64 x 64 blocks, null when every block is admitted.
  const uint8_t* bmask = nullptr;
  int nqb = 0, nkb = 0;
};

struct DecodeArgs {
  const void* q;
  const void* kcache;
  const void* vcache;
  const int32_t* seqlens;
  const int32_t* offsets;       // packed cache (null when paged)
  const int32_t* block_table;   // paged cache: [B, bt_stride] page numbers (null when packed)
  int bt_stride;                // entries per block-table row
  int page_shift;               // log2(page_size)
  int num_pages;                // pages in the pool
  void* o;
  float* lse;
  int B, H, d, max_seqlen;
  float scale;
  int split_keys;  // resolved (> 0)
  int n_splits;    // ceil(max_seqlen / split_keys)
  float* ws;       // chunk states: u [B, H, n_splits, d], then (m, l) [B, H, n_splits, 2]
  // Arrival counters [B * H], zero between calls: the last chunk of a
  // sequence to finish merges (no merge kernel).  Null: a merge kernel runs.
  uint32_t* counters;
  hipStream_t stream;
};

// Backward pass: q, k, v, o, dout bf16 [B, H, N, d]; lse fp32 [B, H, Nq];
// dq, dk, dv fp32 [B, H, N, d]; ws = 2 * B * H * Nq floats.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  float* ws;
  int B, H, Nq, Nk, d;
  float scale;
  int causal;
  hipStream_t stream;
};

hipError_t launch_bwd_bf16(const BwdArgs& a);
long long bwd_bf16_grid(int B, int H, int N);

hipError_t launch_fwd_bf16(const FwdArgs& a);      // d = 128 here, d = 64 below
hipError_t launch_fwd_bf16_d64(const FwdArgs& a);  // fwd_bf16_d64.hip
hipError_t launch_fwd_f32(const FwdArgs& a);
hipError_t launch_decode(const DecodeArgs& a);
// Compute units of the device the stream belongs to (cached per device).
hipError_t cu_count(hipStream_t stream, int* cus);
// Device address of the fixed decode scratch on the stream's device (set up
// on the first call per device).
hipError_t noalloc_scratch(hipStream_t stream, float** ptr);

// Workgroup counts, so the host can reject grids the hardware cannot launch.
long long fwd_bf16_grid(int B, int H, int Nq);
long long fwd_f32_grid(int B, int H, int Nq);

}  // namespace fa
