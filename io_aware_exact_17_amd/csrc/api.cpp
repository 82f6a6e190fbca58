// api.cpp — the C ABI declared in include/fa.h: argument checks (all before
// any HIP call), kernel selection and launch-status mapping.
#include "fa.h"

#include <climits>
#include <cstdint>
#include <cmath>

#include "kernels.hpp"

namespace {

constexpr long long kMaxGridX = 0x7fffffffLL;  // HIP grid.x limit
constexpr long long kMaxGridYZ = 65535;
constexpr long long kPlanChunks = 256;    // chunks per sequence the automatic plan allows
constexpr long long kMaxChunks = 4096;    // chunks per sequence the merge kernel combines
constexpr long long kMaxFusedChunks = 1024;  // ... the last chunk to finish combines
// Calls with more chunk workgroups than this merge in a second kernel: in a
// large grid the last-arriver merge costs more than it saves (every chunk
// then stores its state coherently and waits for the stores before counting
// in: batched 64 x 32 heads, 16384 workgroups, 1445 us against 1429 us for
// split + merge kernel; the single 8192-token request, 1024 workgroups, 31.1
// against 31.0 us, in one process on one box).
constexpr long long kMaxFusedWorkgroups = 4096;
// Every decode workspace starts with this many arrival counters (4 bytes
// each, 64 KiB), zero between calls; chunk states follow.  The region has a
// fixed size so that no call's chunk states ever land on a counter, whatever
// the shapes of earlier calls on the same workspace.
constexpr long long kCounterSlots = 16384;
constexpr size_t kCounterBytes = (size_t)kCounterSlots * 4;
constexpr long long kMaxPageSize = 1 << 16;   // tokens per page of a paged cache
constexpr int kSparseBlock = 64;              // rows and keys per block-sparse mask block
constexpr int kMaxSparseKeyBlocks = 1024;     // key blocks a block-sparse walk may list
constexpr long long kMaxChunkPages = 1024;    // pages one chunk may span (staged in LDS)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Longest sequence any entry point accepts (query or key count, decode
// history).  Kernel index arithmetic is 32-bit; with lengths up to 2^30 every
// position, tile bound and row offset within a head stays far from overflow.
constexpr long long kMaxLen = 1LL << 30;

bool dims_ok(int B, int H, int Nq, int Nk) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return false;
  if (Nq > kMaxLen || Nk > kMaxLen) return false;
  if ((long long)B * H > INT_MAX) return false;
  return true;
}

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

int fwd_common(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int Nq, int Nk, int d, float scale, int causal, hipStream_t stream, bool f32) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
    return FA_ERR_INVALID_ARG;
  if (!dims_ok(B, H, Nq, Nk)) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  const long long grid = f32 ? fa::fwd_f32_grid(B, H, Nq) : fa::fwd_bf16_grid(B, H, Nq);
  if (grid > kMaxGridX) return FA_ERR_INVALID_ARG;
  fa::FwdArgs a{q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal ? 1 : 0, stream};
  const hipError_t e = f32 ? fa::launch_fwd_f32(a) : fa::launch_fwd_bf16(a);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// Chunk size for split-KV decode: start at 256 keys (one workgroup then
// streams 128 KiB of K+V at d=128) and double while the grid would exceed
// 16384 workgroups (64 per CU) or a sequence would have more than 256
// chunks, so a large batch gets fewer, longer chunks; with fewer
// (sequence, head) pairs than CUs, also double while the grid would keep at
// least one workgroup per CU (256 on this device), so each workgroup streams
// a long chunk and few partial states are merged.  Measured: the 64-sequence,
// 32-head batch of lengths up to 16384 reads at 6.34 / 6.42 / 6.38 / 6.23
// TB/s with chunks of 1024 / 2048 / 4096 / 8192 keys; the 8192-token
// request with 32 heads takes 32.2 / 29.5 / 28.4 / 27.0 / 38.2 us with chunks
// of 128 / 256 / 512 / 1024 / 2048 (1024: 8 chunks x 32 heads = 256
// workgroups).
constexpr long long kTargetWorkgroups = 256;
int choose_split_keys(int B, int H, int max_seqlen) {
  const long long bh = (long long)B * H;  // B, H >= 1; B * H * chunks > 16384 <=> chunks > 16384 / bh
  long long sk = 256;
  while (sk < max_seqlen &&
         (ceil_div(max_seqlen, sk) > 16384 / bh || ceil_div(max_seqlen, sk) > kPlanChunks ||
          (bh < kTargetWorkgroups && bh * ceil_div(max_seqlen, 2 * sk) >= kTargetWorkgroups)))
    sk *= 2;
  return (int)sk;
}

// Shapes every decode entry point and sizing function accepts (the grid
// holds H and B in its x and z dimensions; every size product then fits in
// 64 bits).
bool decode_dims_ok(int B, int H, long long max_seqlen) {
  return B >= 1 && H >= 1 && B <= kMaxGridYZ && H <= kMaxGridYZ && max_seqlen >= 1 &&
         max_seqlen <= kMaxLen;
}

bool page_size_ok(int page_size) {
  return page_size >= 1 && page_size <= kMaxPageSize && (page_size & (page_size - 1)) == 0;
}

// Chunk-size constraints every decode launch must meet: a positive multiple
// of 64, at most kMaxChunks chunks per sequence and, for a paged cache, at
// most kMaxChunkPages pages per chunk (a chunk that starts inside a page
// spans one page more than its length needs).
bool chunking_ok(long long max_seqlen, long long sk, int page_size) {
  if (sk < 64 || sk % 64 != 0) return false;
  if ((max_seqlen + sk - 1) / sk > kMaxChunks) return false;
  if (page_size > 0 && (sk + page_size - 1) / page_size + 1 > kMaxChunkPages) return false;
  return true;
}

// The packed plan, halved while a chunk would span more pages than the
// kernel stages in LDS; 0 if no chunk size fits both limits.
int choose_paged_split_keys(int B, int H, int max_seqlen, int page_size) {
  long long sk = choose_split_keys(B, H, max_seqlen);
  while ((sk + page_size - 1) / page_size + 1 > kMaxChunkPages && sk > 64) sk /= 2;
  return chunking_ok(max_seqlen, sk, page_size) ? (int)sk : 0;
}

size_t split_workspace_bytes(int B, int H, int d, long long max_seqlen, long long sk) {
  const long long n_splits = (max_seqlen + sk - 1) / sk;
  // counters, then u[d] per (sequence, head, chunk), then (m, l) per chunk
  return kCounterBytes + (size_t)B * (size_t)H * (size_t)n_splits * (size_t)(d + 2) * sizeof(float);
}

// Launch-time choice between the fused merge (last chunk to finish merges)
// and the separate merge kernel: the fused one needs a counter per (sequence,
// head) inside the fixed counter region.
uint32_t* counters_for(void* workspace, int B, int H, long long n_splits) {
  if ((long long)B * H > kCounterSlots || n_splits > kMaxFusedChunks) return nullptr;
  if ((long long)B * H * n_splits > kMaxFusedWorkgroups) return nullptr;
  return static_cast<uint32_t*>(workspace);
}
float* states_of(void* workspace) {
  return reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes);
}

int decode_packed(const void* q, const void* kcache, const void* vcache, const int32_t* seqlens,
                  const int32_t* offsets, void* o, float* lse, int B, int H, int d, int max_seqlen,
                  float scale, int split_keys, void* workspace, size_t workspace_bytes,
                  hipStream_t stream) {
  if (!q || !kcache || !vcache || !seqlens || !offsets || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned4(o) ||
      !aligned4(lse) || !aligned4(seqlens) || !aligned4(offsets))
    return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || max_seqlen < 1 || max_seqlen > kMaxLen) return FA_ERR_INVALID_ARG;
  if (B > kMaxGridYZ || H > kMaxGridYZ) return FA_ERR_INVALID_ARG;  // grid.z / grid.x
  if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (split_keys < 0) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  const int sk = split_keys > 0 ? split_keys : choose_split_keys(B, H, max_seqlen);
  if (!chunking_ok(max_seqlen, sk, 0)) return FA_ERR_INVALID_ARG;
  const long long n_splits = ((long long)max_seqlen + sk - 1) / sk;
  const size_t need = split_workspace_bytes(B, H, d, max_seqlen, sk);
  if (!workspace || !aligned16(workspace) || workspace_bytes < need) return FA_ERR_WORKSPACE;
  fa::DecodeArgs a{q,  kcache, vcache, seqlens, offsets, nullptr,   0,  0,
                   0,  o,      lse,    B,       H,       d,         max_seqlen, scale,
                   sk, (int)n_splits, states_of(workspace), counters_for(workspace, B, H, n_splits),
                   stream};
  return fa::launch_decode(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

int fa_decode_paged_split_keys(int B, int H, int d, int max_seqlen, int page_size) {
  (void)d;
  if (!decode_dims_ok(B, H, max_seqlen) || !page_size_ok(page_size)) return 0;
  return choose_paged_split_keys(B, H, max_seqlen, page_size);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
           int Nk, int d, float scale, int causal, hipStream_t stream) {
  return fwd_common(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, stream, false);
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
               int Nq, int Nk, int d, float scale, int causal, hipStream_t stream) {
  return fwd_common(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, stream, true);
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B, int H, int d,
                  int total_q, int max_seqlen_q, float scale, int causal, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse) ||
      !aligned4(cu_seqlens_q) || !aligned4(cu_seqlens_k))
    return FA_ERR_INVALID_ARG;
  if (B < 1 || B > kMaxGridYZ || H < 1 || total_q < 1 || max_seqlen_q < 1) return FA_ERR_INVALID_ARG;
  if (max_seqlen_q > kMaxLen) return FA_ERR_INVALID_ARG;
  if ((long long)B * H > INT_MAX) return FA_ERR_INVALID_ARG;
  if (max_seqlen_q > total_q) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // d = 128: grid = (query tiles of the longest sequence x H, B); d = 64: one
  // workgroup per (sequence, query tile, head) item, counted over the whole
  // batch.  Same tile height as dense.
  if (fa::fwd_bf16_grid(d == 64 ? B : 1, H, max_seqlen_q) > kMaxGridX) return FA_ERR_INVALID_ARG;
  fa::FwdArgs a{q, k, v, o, lse, B, H, max_seqlen_q, 0, d, scale, causal ? 1 : 0, stream};
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.total_q = total_q;
  return fa::launch_fwd_bf16(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                        const uint8_t* block_mask, int B, int H, int Nq, int Nk, int d,
                        float scale, int causal, hipStream_t stream) {
  if (!block_mask) return FA_ERR_INVALID_ARG;
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
    return FA_ERR_INVALID_ARG;
  if (!dims_ok(B, H, Nq, Nk)) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  if (ceil_div(Nk, kSparseBlock) > kMaxSparseKeyBlocks) return FA_ERR_INVALID_ARG;
  if (fa::fwd_bf16_grid(B, H, Nq) > kMaxGridX) return FA_ERR_INVALID_ARG;
  fa::FwdArgs a{q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal ? 1 : 0, stream};
  a.bmask = block_mask;
  a.nqb = (int)ceil_div(Nq, kSparseBlock);
  a.nkb = (int)ceil_div(Nk, kSparseBlock);
  return fa::launch_fwd_bf16(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_bytes(int B, int H, int Nq) {
  if (B < 1 || H < 1 || Nq < 1) return 0;
  return 2 * (size_t)B * (size_t)H * (size_t)Nq * sizeof(float);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, float* dq, float* dk, float* dv, int B, int H, int Nq, int Nk, int d,
           float scale, int causal, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned4(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_INVALID_ARG;
  if (!dims_ok(B, H, Nq, Nk)) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (fa::bwd_bf16_grid(B, H, Nq) > kMaxGridX || fa::bwd_bf16_grid(B, H, Nk) > kMaxGridX)
    return FA_ERR_INVALID_ARG;
  if ((long long)B * H * Nq > (long long)kMaxGridX * 16) return FA_ERR_INVALID_ARG;  // row pass grid
  const size_t need = fa_bwd_workspace_bytes(B, H, Nq);
  if (!workspace || !aligned16(workspace) || workspace_bytes < need) return FA_ERR_WORKSPACE;
  fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, static_cast<float*>(workspace),
                B, H, Nq, Nk, d, scale, causal ? 1 : 0, stream};
  return fa::launch_bwd_bf16(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_decode_split_keys(int B, int H, int d, int max_seqlen) {
  (void)d;
  if (!decode_dims_ok(B, H, max_seqlen)) return 0;
  return choose_split_keys(B, H, max_seqlen);
}

size_t fa_decode_split_workspace_bytes(int B, int H, int d, int max_seqlen, int split_keys) {
  if (!decode_dims_ok(B, H, max_seqlen) || (d != 64 && d != 128) || split_keys < 0) return 0;
  const long long sk = split_keys > 0 ? split_keys : choose_split_keys(B, H, max_seqlen);
  if (!chunking_ok(max_seqlen, sk, 0)) return 0;
  return split_workspace_bytes(B, H, d, max_seqlen, sk);
}

size_t fa_decode_workspace_bytes(int B, int H, int d, int max_seqlen) {
  return fa_decode_split_workspace_bytes(B, H, d, max_seqlen, 0);
}

int fa_decode_varlen(const void* q, const void* kcache, const void* vcache, const int32_t* seqlens,
                     const int32_t* offsets, void* o, float* lse, int B, int H, int d,
                     int max_seqlen, float scale, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  return decode_packed(q, kcache, vcache, seqlens, offsets, o, lse, B, H, d, max_seqlen, scale, 0,
                       workspace, workspace_bytes, stream);
}

int fa_decode_varlen_split(const void* q, const void* kcache, const void* vcache,
                           const int32_t* seqlens, const int32_t* offsets, void* o, float* lse,
                           int B, int H, int d, int max_seqlen, float scale, int split_keys,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (split_keys < 1) return FA_ERR_INVALID_ARG;
  return decode_packed(q, kcache, vcache, seqlens, offsets, o, lse, B, H, d, max_seqlen, scale,
                       split_keys, workspace, workspace_bytes, stream);
}

int fa_decode_paged(const void* q, const void* kpages, const void* vpages,
                    const int32_t* block_table, const int32_t* seqlens, void* o, float* lse, int B,
                    int H, int d, int page_size, int num_pages, int max_blocks, int max_seqlen,
                    float scale, int split_keys, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  if (!q || !kpages || !vpages || !block_table || !seqlens || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(kpages) || !aligned16(vpages) || !aligned4(o) ||
      !aligned4(lse) || !aligned4(seqlens) || !aligned4(block_table))
    return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || max_seqlen < 1 || num_pages < 1 || max_blocks < 1) return FA_ERR_INVALID_ARG;
  if (max_seqlen > kMaxLen) return FA_ERR_INVALID_ARG;
  if (B > kMaxGridYZ || H > kMaxGridYZ) return FA_ERR_INVALID_ARG;  // grid.z / grid.x
  if (!page_size_ok(page_size)) return FA_ERR_INVALID_ARG;
  if ((long long)max_blocks * page_size < max_seqlen) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (split_keys < 0) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  const long long sk = split_keys > 0 ? split_keys : choose_paged_split_keys(B, H, max_seqlen, page_size);
  if (!chunking_ok(max_seqlen, sk, page_size)) return FA_ERR_INVALID_ARG;
  const long long n_splits = ((long long)max_seqlen + sk - 1) / sk;
  const size_t need = split_workspace_bytes(B, H, d, max_seqlen, sk);
  if (!workspace || !aligned16(workspace) || workspace_bytes < need) return FA_ERR_WORKSPACE;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  fa::DecodeArgs a{q,  kpages, vpages,     seqlens, nullptr, block_table, max_blocks, shift,
                   num_pages, o, lse,      B,       H,       d,           max_seqlen, scale,
                   (int)sk, (int)n_splits, states_of(workspace),
                   counters_for(workspace, B, H, n_splits), stream};
  return fa::launch_decode(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_decode_varlen_noalloc(const void* q, const void* kcache, const void* vcache,
                             const int32_t* seqlens, const int32_t* offsets, void* o, float* lse,
                             int B, int H, int d, int max_seqlen, float scale, hipStream_t stream) {
  if (!q || !kcache || !vcache || !seqlens || !offsets || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned4(o) ||
      !aligned4(lse) || !aligned4(seqlens) || !aligned4(offsets))
    return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || max_seqlen < 1 || max_seqlen > kMaxLen) return FA_ERR_INVALID_ARG;
  if (B > kMaxGridYZ || H > kMaxGridYZ) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  const int sk = choose_split_keys(B, H, max_seqlen);
  if (!chunking_ok(max_seqlen, sk, 0)) return FA_ERR_INVALID_ARG;
  const long long n_splits = ((long long)max_seqlen + sk - 1) / sk;
  // chunk states only: this path merges with the merge kernel, no counters
  const size_t need = (size_t)B * (size_t)H * (size_t)n_splits * (size_t)(d + 2) * sizeof(float);
  if (need > (size_t)FA_DECODE_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  float* ws = nullptr;
  if (fa::noalloc_scratch(stream, &ws) != hipSuccess) return FA_ERR_HIP;
  fa::DecodeArgs a{q,  kcache, vcache, seqlens, offsets, nullptr, 0, 0,
                   0,  o,      lse,    B,       H,       d,       max_seqlen, scale,
                   sk, (int)n_splits, ws, nullptr, stream};
  return fa::launch_decode(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dimension must be 64 or 128";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime refused the launch";
    case FA_ERR_SCRATCH:
      return "FA_ERR_SCRATCH: the call needs more than the fixed scratch of fa_decode_varlen_noalloc";
    default: return "unknown fa_status";
  }
}

}  // extern "C"
