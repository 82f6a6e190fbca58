// decode.hip — single-query attention over a packed variable-length KV cache.
//
// With one new query per sequence the score row is 1 x history and there is
// no N x N matrix; the cost is reading the cached keys and values (and, for a
// single request, the launch itself): FlashAttention explainer
// (cztcode.com/2026/5368) §6.  These are bandwidth kernels: no matrix cores,
// 16-byte loads, two batches of loads in flight per lane, enough workgroups
// to cover every CU even for one sequence, and a merge built from parallel
// loads so that it costs a few memory latencies.
//
// Each sequence's keys are cut into chunks of `split_keys`.  A workgroup of
// the split kernel streams one (head, chunk, sequence): every key row (d bf16
// = 256 B at d=128) is read by a group of d/8 lanes, 16 bytes each; the q.k
// dot product is finished with DPP row reductions; each lane group keeps the
// running state (m, l, u) of the explainer's §2 recurrence, updated once per
// batch of keys; the lane groups are merged through LDS with the block-merge
// rule of explainer §3/§7 (m = max, l and u rescaled by exp(m_i - m) and
// added).  A sequence that fits in one chunk is finished on the spot;
// otherwise the chunk's state goes to the workspace and the merge kernel
// combines a sequence's chunk states with the same rule, writing O = u / l
// and LSE = m + ln l.  Cache row addresses are 64-bit.
#include <mutex>

#include "cdna4.hpp"
#include "fa.h"
#include "kernels.hpp"

// Fixed scratch for fa_decode_varlen_noalloc (callers that cannot allocate):
// one copy per device, alive until the process ends.  Host code never uses
// this name as an address; it uses the per-device pointer from
// hipGetSymbolAddress (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[FA_DECODE_NOALLOC_SCRATCH_BYTES];

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunkPages = 1024;  // pages one chunk may span (paged cache)
constexpr int kMaxChunks = 4096;      // chunks per sequence the merge kernel combines

template <int D>
struct DecCfg {
  static constexpr int LPR = D / 8;           // lanes per key row (16 B each)
  static constexpr int NRG = kThreads / LPR;  // key rows covered per pass
  // keys per lane group per batch: 4 at d = 128 keeps the kernel at ~100
  // vector registers, so four workgroups share a CU and the single request's
  // 1024 chunks all run at once (30.6 -> 30.0 us against 8 keys)
  static constexpr int U = D == 128 ? 4 : 8;
};

template <int D>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (D == 128) return sum_row16(x);
  else return sum_row8(x);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Device-coherent 8-byte store / load (relaxed, agent scope): they bypass
// the per-XCD L2, so a workgroup on another XCD reads what the writer stored
// once the writer's store has completed.
__device__ __forceinline__ void store_coherent(float* p, float a, float b) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, f32x2{a, b}),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <bool COHERENT>
__device__ __forceinline__ f32x2 load_state(const float* p) {
  if constexpr (COHERENT)
    return __builtin_bit_cast(f32x2, __hip_atomic_load(reinterpret_cast<const uint64_t*>(p),
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  else
    return *reinterpret_cast<const f32x2*>(p);
}

// Merge n >= 2 chunk states of one (sequence, head) with the block-merge
// rule (explainer §3/§7) and write O = u / l (bf16) and LSE = m + ln l.
// ml holds (m, l) per chunk (m in log2 units), u the unnormalised u[D] per
// chunk.  Run by the first NW waves of the workgroup (threads 0 .. 64 NW - 1);
// sm_cm / sm_cl hold one float per chunk; sm_red and sm_part are used when
// NW > 1.  All (m, l) pairs are requested at once (64 NW per round), then the
// waves split the chunks for the u sums (two dims per lane, eight loads in
// flight), so the merge costs a few memory latencies, not one per chunk.
template <int D, int NW, bool COHERENT>
__device__ __forceinline__ void merge_chunks(const float* __restrict__ u, const float* __restrict__ ml,
                                             int n, bf16* __restrict__ o_row,
                                             float* __restrict__ lse_out, float* sm_cm, float* sm_cl,
                                             float (*sm_red)[NW], float (*sm_part)[D]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float mloc = kNegInf;
  for (int t = tid; t < n; t += 64 * NW) {
    const f32x2 x = load_state<COHERENT>(ml + 2 * (size_t)t);
    sm_cm[t] = x[0];
    sm_cl[t] = x[1];
    mloc = fmaxf(mloc, x[0]);
  }
  float M = wave_max(mloc);
  if constexpr (NW > 1) {
    if (lane == 0) sm_red[0][wave] = M;
    __syncthreads();
    M = sm_red[0][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm_red[0][w]);
  }
  // Each thread turns its own chunks' m into the factor 2^(m - M).
  float lloc = 0.f;
  for (int t = tid; t < n; t += 64 * NW) {
    const float f = exp2_hw(sm_cm[t] - M);
    sm_cm[t] = f;
    lloc = __builtin_fmaf(f, sm_cl[t], lloc);
  }
  float L = wave_sum(lloc);
  if constexpr (NW > 1) {
    if (lane == 0) sm_red[1][wave] = L;
    __syncthreads();  // also orders the factors in sm_cm before the reads below
    L = sm_red[1][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) L += sm_red[1][w];
  }
  const int d0 = 2 * lane;
  float G0 = 0.f, G1 = 0.f;
  if (d0 < D) {
#pragma unroll 8
    for (int t = wave; t < n; t += NW) {
      const f32x2 w = load_state<COHERENT>(u + (size_t)t * D + d0);
      G0 = __builtin_fmaf(sm_cm[t], w[0], G0);
      G1 = __builtin_fmaf(sm_cm[t], w[1], G1);
    }
  }
  if constexpr (NW > 1) {
    if (d0 < D) {
      sm_part[wave][d0] = G0;
      sm_part[wave][d0 + 1] = G1;
    }
    __syncthreads();
    if (wave != 0) return;
    if (d0 < D) {
      G0 = sm_part[0][d0];
      G1 = sm_part[0][d0 + 1];
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        G0 += sm_part[w][d0];
        G1 += sm_part[w][d0 + 1];
      }
    }
  }
  const float inv = 1.f / L;
  if (d0 < D) *reinterpret_cast<uint32_t*>(o_row + d0) = pack_bf16x2(G0 * inv, G1 * inv);
  if (lane == 0) *lse_out = (M + log2_hw(L)) * kLn2;
}

// The merge done by the last chunk of a (sequence, head) to finish, one
// wave: the n >= 2 chunk states are taken 32 at a time, each group in one
// memory round trip (lane i loads chunk i's (m, l); every lane loads the u
// values of its two dims for all 32 chunks at once), and the groups are
// combined with the block-merge rule as they come.  Chunk i's factor
// 2^(m_i - M) is read from lane i.  Writes O = u / l (bf16) and LSE.
template <int D>
__device__ __forceinline__ void merge_last_arriver(const float* __restrict__ u,
                                                   const float* __restrict__ ml, int n,
                                                   bf16* __restrict__ o_row, float* __restrict__ lse_out) {
  constexpr int kGroup = 32;
  const int lane = threadIdx.x & 63;
  const int d0 = 2 * lane;
  const bool has_d = d0 < D;
  float M = kNegInf, L = 0.f, G0 = 0.f, G1 = 0.f;
  for (int base = 0; base < n; base += kGroup) {
    const int cnt = min(kGroup, n - base);
    const f32x2 x = lane < cnt ? load_state<true>(ml + 2 * (size_t)(base + lane)) : f32x2{kNegInf, 0.f};
    f32x2 w[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i)
      w[i] = (i < cnt && has_d) ? load_state<true>(u + (size_t)(base + i) * D + d0) : f32x2{0.f, 0.f};
    const float m_new = fmaxf(M, wave_max(x[0]));
    const float alpha = exp2_hw(M - m_new);  // 0 while M = -inf
    const float f = exp2_hw(x[0] - m_new);   // this lane's chunk factor (0 for no chunk)
    L = __builtin_fmaf(L, alpha, wave_sum(f * x[1]));
    G0 *= alpha;
    G1 *= alpha;
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const float fi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), i));
      G0 = __builtin_fmaf(fi, w[i][0], G0);
      G1 = __builtin_fmaf(fi, w[i][1], G1);
    }
    M = m_new;
  }
  const float inv = 1.f / L;
  if (has_d) *reinterpret_cast<uint32_t*>(o_row + d0) = pack_bf16x2(G0 * inv, G1 * inv);
  if (lane == 0) *lse_out = (M + log2_hw(L)) * kLn2;
}

// PAGED: the cache is a pool of pages [num_pages, page_size, H, d] and
// sequence b's key t lives in page block_table[b][t / page_size], slot
// t % page_size (page_size a power of two); otherwise the cache is packed
// and sequence b owns rows offsets[b] ...
//
// FUSED: the chunks of a sequence that spans several are merged by the last
// of them to finish, found through counters[b * H + h] (zero between calls).
template <int D, bool PAGED, bool FUSED>
__global__ __launch_bounds__(kThreads, 2) void decode_split_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
    const int32_t* __restrict__ seqlens, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ block_table, int bt_stride, int page_shift, int num_pages,
    bf16* __restrict__ O, float* __restrict__ LSE, float* __restrict__ ws_u,
    float* __restrict__ ws_ml, uint32_t* __restrict__ counters, int H, int split_keys,
    int n_splits, float c) {
  using C = DecCfg<D>;
  // Heads vary fastest across the grid, so the workgroups running together
  // read neighbouring 256-byte head slices of the same token rows.
  const int h = blockIdx.x, s = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int len = seqlens[b];
  const size_t bh = (size_t)b * H + h;
  if (len <= 0) {  // empty history: O = 0, LSE = -inf
    if (s == 0) {
      if (tid < D / 2) *reinterpret_cast<uint32_t*>(O + bh * D + 2 * tid) = 0u;
      if (tid == 0) LSE[bh] = kNegInf;
    }
    return;
  }
  const int k_begin = s * split_keys;
  if (k_begin >= len) return;  // chunk past this sequence's end
  const int k_end = min(len, k_begin + split_keys);
  const int n_active = min(n_splits, (len + split_keys - 1) / split_keys);
  // Cache row of the sequence's key kk.  Paged: the chunk's page numbers are
  // staged in LDS once (entries out of range read the last page instead of
  // faulting), then every key costs an LDS read, a shift and an add.
  __shared__ int sm_page[PAGED ? kMaxChunkPages : 1];
  size_t base = 0;
  int p0 = 0;
  if constexpr (PAGED) {
    p0 = k_begin >> page_shift;
    const int np = ((k_end - 1) >> page_shift) - p0 + 1;
    const int32_t* bt = block_table + (size_t)b * bt_stride + p0;
    for (int i = tid; i < np; i += kThreads)
      sm_page[i] = (int)min((unsigned)bt[i], (unsigned)(num_pages - 1));
    __syncthreads();
  } else {
    base = (size_t)offsets[b];
  }
  const int page_mask = (1 << page_shift) - 1;
  auto row_of = [&](int kk) -> size_t {
    if constexpr (PAGED)
      return ((size_t)sm_page[(kk >> page_shift) - p0] << page_shift) + (size_t)(kk & page_mask);
    else
      return base + (size_t)kk;
  };

  const int sub = tid % C::LPR;  // which 8 dims of the row this lane reads
  const int rg = tid / C::LPR;   // lane group

  float qv[8];
  {
    const u32x4 w = *reinterpret_cast<const u32x4*>(q + bh * D + sub * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qv[2 * i] = bf16_lo(w[i]);
      qv[2 * i + 1] = bf16_hi(w[i]);
    }
  }

  const size_t row_stride = (size_t)H * D;
  const bf16* kp = kc + (size_t)h * D + sub * 8;
  const bf16* vp = vc + (size_t)h * D + sub * 8;

  float m = kNegInf, l = 0.f;
  float u[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) u[e] = 0.f;

  // Batch t covers keys k_begin + rg + NRG*(U*t + i), i < U.  Two batches of
  // loads are in flight: the next one is issued before the current one is
  // consumed.  Keys past k_end read the chunk's first key (in range, finite)
  // and are given score -inf.  Every cache byte is read once per call, so the
  // loads carry the non-temporal hint (about 9% more bandwidth than plain
  // loads on both decode workloads).
  constexpr int kStep = C::NRG * C::U;
  u32x4 kA[C::U], vA[C::U], kB[C::U], vB[C::U];
  auto load = [&](u32x4 (&kr)[C::U], u32x4 (&vr)[C::U], int k0) {
#pragma unroll
    for (int i = 0; i < C::U; ++i) {
      int kk = k0 + C::NRG * i;
      kk = kk < k_end ? kk : k_begin;
      const size_t row = row_of(kk);
      kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + row * row_stride));
      vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + row * row_stride));
    }
  };
  auto consume = [&](const u32x4 (&kr)[C::U], const u32x4 (&vr)[C::U], int k0) {
    float sc[C::U];
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < C::U; ++i) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        part = __builtin_fmaf(qv[2 * e], bf16_lo(kr[i][e]), part);
        part = __builtin_fmaf(qv[2 * e + 1], bf16_hi(kr[i][e]), part);
      }
      const float dot = row_sum<D>(part);
      sc[i] = (k0 + C::NRG * i < k_end) ? dot * c : kNegInf;
      mx = fmaxf(mx, sc[i]);
    }
    if (mx == kNegInf) return;  // no key of this batch for this lane group
    const float m_new = fmaxf(m, mx);
    const float alpha = exp2_hw(m - m_new);  // 0 while m = -inf
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) u[e] *= alpha;
#pragma unroll
    for (int i = 0; i < C::U; ++i) {
      const float p = exp2_hw(sc[i] - m_new);
      l += p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u[2 * e] = __builtin_fmaf(p, bf16_lo(vr[i][e]), u[2 * e]);
        u[2 * e + 1] = __builtin_fmaf(p, bf16_hi(vr[i][e]), u[2 * e + 1]);
      }
    }
    m = m_new;
  };

  const int k_first = k_begin + rg;
  if (k_first < k_end) {
    load(kA, vA, k_first);
    for (int k0 = k_first;; k0 += 2 * kStep) {
      const bool more1 = k0 + kStep < k_end;
      if (more1) load(kB, vB, k0 + kStep);
      consume(kA, vA, k0);
      if (!more1) break;
      const bool more2 = k0 + 2 * kStep < k_end;
      if (more2) load(kA, vA, k0 + 2 * kStep);
      consume(kB, vB, k0 + kStep);
      if (!more2) break;
    }
  }

  // Merge the lane groups' states (block-merge rule) through LDS; wave 0
  // finishes the chunk, each of its lanes owning dims 2*lane and 2*lane+1.
  __shared__ float sm_m[C::NRG], sm_l[C::NRG];
  __shared__ float sm_u[C::NRG][D + 4];
  if (sub == 0) {
    sm_m[rg] = m;
    sm_l[rg] = l;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) sm_u[rg][sub * 8 + e] = u[e];
  __syncthreads();
  if (tid >= 64) return;
  const int lane = tid;
  const int d0 = 2 * lane;
  const bool has_d = d0 < D;
  float M = kNegInf, L = 0.f, U0 = 0.f, U1 = 0.f;
  for (int g = 0; g < C::NRG; ++g) M = fmaxf(M, sm_m[g]);
  for (int g = 0; g < C::NRG; ++g) {
    const float f = exp2_hw(sm_m[g] - M);  // empty groups (m = -inf) weigh 0
    L = __builtin_fmaf(f, sm_l[g], L);
    if (has_d) {
      U0 = __builtin_fmaf(f, sm_u[g][d0], U0);
      U1 = __builtin_fmaf(f, sm_u[g][d0 + 1], U1);
    }
  }

  if (n_active == 1) {  // the whole history was this chunk
    const float inv = 1.f / L;
    if (has_d) *reinterpret_cast<uint32_t*>(O + bh * D + d0) = pack_bf16x2(U0 * inv, U1 * inv);
    if (lane == 0) LSE[bh] = (M + log2_hw(L)) * kLn2;
    return;
  }

  // Leave this chunk's state (u[D], then (m, l)) for the merge.
  const size_t slot = bh * n_splits + s;
  if constexpr (!FUSED) {
    if (has_d) *reinterpret_cast<f32x2*>(ws_u + slot * D + d0) = f32x2{U0, U1};
    if (lane == 0) *reinterpret_cast<f32x2*>(ws_ml + slot * 2) = f32x2{M, L};
  } else {
    if (has_d) store_coherent(ws_u + slot * D + d0, U0, U1);
    if (lane == 0) store_coherent(ws_ml + slot * 2, M, L);
    // The state has reached the coherence point before the arrival counts.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    uint32_t seen = 0;
#ifdef FA_PARANOID_SYNC
    // race-check build: full device-scope release / acquire around the count
    __threadfence();
    if (lane == 0)
      seen = __hip_atomic_fetch_add(counters + bh, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    __threadfence();
#else
    if (lane == 0)
      seen = __hip_atomic_fetch_add(counters + bh, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#endif
    seen = __builtin_amdgcn_readfirstlane(seen);
    if (seen != (uint32_t)(n_active - 1)) return;  // another chunk is still running
    // Last to arrive: every other chunk's state is in place.  Reset the
    // counter for the next call, then merge.
    if (lane == 0) __hip_atomic_store(counters + bh, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    merge_last_arriver<D>(ws_u + bh * n_splits * D, ws_ml + bh * n_splits * 2, n_active, O + bh * D,
                          LSE + bh);
  }
}

// One 256-thread workgroup per (sequence, head) merges the chunk states of
// sequences that did not fit in one chunk (the others were finished by the
// split kernel).
template <int D>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(
    const float* __restrict__ ws_u, const float* __restrict__ ws_ml,
    const int32_t* __restrict__ seqlens, bf16* __restrict__ O, float* __restrict__ LSE, int H,
    int split_keys, int n_splits) {
  constexpr int NW = kThreads / 64;
  const int h = blockIdx.x, b = blockIdx.y;
  const size_t bh = (size_t)b * H + h;
  __shared__ float sm_cm[kMaxChunks], sm_cl[kMaxChunks];
  __shared__ float sm_red[2][NW];
  __shared__ float sm_part[NW][D];
  const int len = seqlens[b];
  const int n = min(n_splits, len > 0 ? (len + split_keys - 1) / split_keys : 0);
  if (n <= 1) return;  // empty or finished by the split kernel
  merge_chunks<D, NW, false>(ws_u + bh * n_splits * D, ws_ml + bh * n_splits * 2, n, O + bh * D,
                             LSE + bh, sm_cm, sm_cl, sm_red, sm_part);
}

template <int D, bool PAGED, bool FUSED>
hipError_t launch(const DecodeArgs& a) {
  const float c = a.scale * kLog2e;
  float* ws_u = a.ws;
  float* ws_ml = ws_u + (size_t)a.B * a.H * a.n_splits * D;
  {
    void* args[] = {(void*)&a.q,          (void*)&a.kcache,     (void*)&a.vcache,
                    (void*)&a.seqlens,    (void*)&a.offsets,    (void*)&a.block_table,
                    (void*)&a.bt_stride,  (void*)&a.page_shift, (void*)&a.num_pages,
                    (void*)&a.o,          (void*)&a.lse,        (void*)&ws_u,
                    (void*)&ws_ml,        (void*)&a.counters,   (void*)&a.H,
                    (void*)&a.split_keys, (void*)&a.n_splits,   (void*)&c};
    const hipError_t e = hipLaunchKernel(
        reinterpret_cast<const void*>(&decode_split_kernel<D, PAGED, FUSED>),
        dim3((unsigned)a.H, (unsigned)a.n_splits, (unsigned)a.B), dim3(kThreads), args, 0, a.stream);
    if (e != hipSuccess) return e;
  }
  // every sequence finished in the split kernel (one chunk, or merged by its last chunk)
  if (a.n_splits == 1 || FUSED) return hipSuccess;
  void* args[] = {(void*)&ws_u, (void*)&ws_ml, (void*)&a.seqlens, (void*)&a.o, (void*)&a.lse,
                  (void*)&a.H, (void*)&a.split_keys, (void*)&a.n_splits};
  return hipLaunchKernel(reinterpret_cast<const void*>(&decode_merge_kernel<D>),
                         dim3((unsigned)a.H, (unsigned)a.B), dim3(kThreads), args, 0, a.stream);
}

template <int D, bool PAGED>
hipError_t launch_sel(const DecodeArgs& a) {
  return a.counters ? launch<D, PAGED, true>(a) : launch<D, PAGED, false>(a);
}

constexpr int kMaxScratchDevices = 64;

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, float** ptr) {
  static void* table[kMaxScratchDevices];
  static std::mutex lock;
  hipDevice_t dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(lock);
  if (!table[dev]) {
    // Set-up, once per device, with that device current: the device address
    // of this device's copy of `scratch`.
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    table[dev] = p;
  }
  *ptr = static_cast<float*>(table[dev]);
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a) {
  if (a.block_table)
    return a.d == 128 ? launch_sel<128, true>(a) : launch_sel<64, true>(a);
  return a.d == 128 ? launch_sel<128, false>(a) : launch_sel<64, false>(a);
}

}  // namespace fa
